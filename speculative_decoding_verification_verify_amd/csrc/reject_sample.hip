// Lossless rejection-sampling verifier over the full vocabulary, plus the
// commit of the logical KV length, for a draft chain and for a draft tree.
//
// Method: AI Engineering from Scratch, "Speculative decoding and EAGLE-3" --
// "Concept" (accept d ~ p with probability min(1, q(d)/p(d)); on rejection
// draw from (q - p)_+ normalised; bonus token from q_{N+1} when every draft
// passes), "Build it" steps 1-2 (p(d) <= 0 accepts; a zero-mass residual falls
// back to q) and "Rolling back the KV cache" (logical length reset).  Trees:
// the same page's EAGLE-2 draft tree and thakicloud, "Grading every branch in
// one pass": every branch is graded in the one pass and the surviving path is
// kept; the siblings of a node are tried one after another by recursive
// rejection sampling, which keeps the output law exact.
//
// Two kernels on the caller's stream for the chain (three with top-k / top-p,
// whose k_filter runs between the sweep and the decision; a third, k_locate,
// takes the draw when V > 2^19):
//   k_sweep     one pass over every logit row (the HBM-bound part): per 4096-
//               entry chunk, the raw maximum and sum_v 2^(x_v c - m) in fp32
//               (c = log2(e) / T), or the chunk argmax for greedy sequences.
//               One wave per chunk, 16-byte nontemporal loads (1 KB
//               contiguous per instruction), butterfly reductions, no LDS.
//               These statistics feed the accept tests, whose decisions are
//               only sensitive at the 1e-5 level.  The wave whose chunk holds
//               a row's drafted token also records that token's logit.
//   k_decide_residual  per (sequence, 8192-entry chunk), in two steps.
//               The decision: merge the row statistics in a fixed order (16
//               lanes per row, DPP steps), run
//               the K accept tests in parallel on the recorded logits and
//               take the first rejection (every block of the sequence takes
//               the same decision; its first block finishes a greedy
//               sequence, or records the decision for the draw).  Then the
//               pass: summarise this chunk of the one row pair the final
//               draw needs (target and draft row n, or target row K for the
//               bonus) in float64, per 256-entry sub-chunk and per chunk:
//               sum e_q, sum e_p and the same two sums over the entries with
//               q > c p, with e = 2^((x - xmax) c) to a few ulp.  They give
//               the exact normalisers and residual masses, so the row pair is
//               read only once more.
//   the draw   in the workgroup that completes a sampling sequence's pass:
//               float64 prefix scans over the chunk masses, then the
//               sub-chunk masses, then one 256-entry run of exact weights;
//               emit the tokens and commit kv_len.
// The final draw's weights are exact to 2e-13 relative, so the draw agrees
// with a float64 reference except within ~1e-12 of probability mass around
// the CDF edges.  The pass workgroups hand their sums to the one that draws
// without device-scope fences (see the hand-off helpers below).
//
// Tree: the same sweep over the target rows of all nodes and the draft rows
// of the nodes with children; k_tree_decide walks down from the root while
// the first child of each node passes its test (greedy sequences finish
// there).  After a rejection the next sibling is tested against the residual
// q' = (q - coef p)_+ / Z, where coef starts at 1 and grows by Z with every
// further rejection; Z needs one exact pass over the node's row pair (the
// chain's pass).  So the tree runs in rounds of k_tree_round, each round one
// such pass per sequence that still needs one, followed in the same kernel
// by the step after it (run by the workgroup that completes the sequence's
// pass, from chunk sums handed over without fences, as below); the host
// knows from the tree's shape how many rounds the longest walk can take.
// With one tree per sequence (parents on the device), k_tree_shapes first
// builds each sequence's shape in the workspace, the kernels read it from
// there, and the host launches the most rounds an N-node tree can need.
// No floating-point atomics and fixed reduction orders: results are bitwise
// reproducible run to run.

// Contraction off: merges must stay symmetric in their operands, and the
// weights of the draw must equal those of the pass bit for bit.  Fused
// multiply-adds that are wanted are written out.
#pragma clang fp contract(off)

#include <algorithm>
#include <cstddef>
#include <mutex>

#include "common.h"
#include "validate.h"

namespace sv {

constexpr int kThreads = 256;
constexpr int kDecideThreads = 1024;  // tree decision: 16 lanes per row statistic merge
#ifndef SV_SWEEP_CHUNK
#define SV_SWEEP_CHUNK 4096
#endif
constexpr int kSweepChunk = SV_SWEEP_CHUNK;   // entries per wave in k_sweep
constexpr int kResChunk = 8192;       // entries per block of a residual pass
constexpr int kMaxRows = 2 * SV_MAX_K + 1;
constexpr double kLog2eD = 1.4426950408889634074;


// One exact pass over a row pair (and the draw that may follow it), as the
// decide and step kernels leave it for the next pass.
enum : int {
  kModeNone = 0,    // nothing to do: greedy or finished
  kModeQ = 1,       // target row only: the draw is from q (bonus token)
  kModeResid = 2,   // target and draft row: weights (q - coef p)_+
  kModePending = 3, // tree: the walk has ended; its draw (from the pass the
                    // decision describes, mode in draw_mode) waits for k_tree_draw
};
struct Decision {
  int mode;
  int n;             // chain: accepted drafts
  int trow, drow;    // row indices into the target / draft arrays (drow unused in kModeQ)
  float xmq, xmp;    // raw maxima of those rows: the exp frames of the pass
  double theta;      // log2(coef sq / sp): q > coef p iff aq - ap > theta
  double coef;       // residual coefficient (1 after the first rejection at a node)
  double coef_prev;  // the one before it: a zero-mass residual leaves the law at
                     // (q - coef_prev p)_+, which is then q (coef_prev = 0) or p
  uint32_t kq, kp;   // top-k / top-p filters: entries whose order key is below
                     // these weigh 0 (0: no filter)
  int draw_mode;     // kModePending: the mode of the pass the draw is taken from
};

// ---- Top-k / top-p filters (readings: logits / T, then top-k, then top-p
// over the top-k set, each a threshold on the logit value with ties kept).
// Order keys: unsigned integers that sort like the logits (bf16: 16 bits,
// fp32: 32 bits); -inf has the smallest key but one, so key 0 never occurs
// and 0 can mean "no filter".
__host__ __device__ inline uint32_t order_key16(uint32_t h) {
  h = (h == 0x8000u) ? 0u : h;                              // -0 ties with +0
  return (h & 0x8000u) ? (~h & 0xFFFFu) : (h | 0x8000u);
}
__host__ __device__ inline uint32_t order_key32(uint32_t u) {
  u = (u == 0x80000000u) ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// 32-bit key of a float: order_key32, written as a sign-dependent xor plus
// the -0 fix.  For a widened bf16 logit its top 16 bits are order_key16 of
// the bf16 bits.
__device__ __forceinline__ uint32_t key32_of(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t k = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
  return k == 0x7FFFFFFFu ? 0x80000000u : k;
}
// Key of a logit held as a float (a bf16 logit widened exactly, or fp32).
__device__ __forceinline__ uint32_t float_key(float x, bool key16) {
  const uint32_t k = key32_of(x);
  return key16 ? k >> 16 : k;
}

// The float with a given 32-bit key (no NaN keys are passed).
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
constexpr uint32_t kKeyNegInf = 0x007FFFFFu, kKeyPosInf = 0xFF800000u;
// Float bounds [flo, fhi] with  flo <= x <= fhi  <=>  klo <= key32_of(x) <= khi
// for every non-NaN x.  Key 0x7FFFFFFF (-0 before the fix) never occurs, so
// as a bound it is moved past -0: x = -0 compares equal to +0.
__device__ __forceinline__ void key_bounds(uint32_t klo, uint32_t khi, float& flo, float& fhi) {
  klo = max(klo, kKeyNegInf);
  khi = min(khi, kKeyPosInf);
  if (klo == 0x7FFFFFFFu) klo = 0x80000000u;
  if (khi == 0x7FFFFFFFu) khi = 0x7FFFFFFEu;
  flo = key_value(klo);
  fhi = key_value(khi);
}

// What k_filter leaves per row: the kept set {key >= key_min} and its mass
// in the sweep's frame, sum 2^(x c - fl(xmax c)).
struct RowFilter {
  uint32_t key_min;  // 0: the row is not filtered
  uint32_t pad;
  double mass;
};

// The window a filtered sweep counts (bf16 rows of sampling sequences with
// a top-k or top-p filter): consecutive 16-bit keys (the keys of one binade
// of bf16 values are 128 in a row), placed from the largest entry of
// kWinLines 64-entry runs spread evenly over the row (every sweep block of
// the row reads the same runs and derives the same window):
//  * top-k (with or without top-p): kWinKeys keys, from kWinKBelow keys under
//    the sample's largest entry (k up to V / 256; all kWinKeys keys for
//    larger k) to kWinTopMargin keys above it.
//  * top-p alone: kWinPKeys keys up to kWinPTopMargin keys above the
//    sample's largest entry, so six binades under it.  A top-p threshold
//    lies under the bulk of the row's mass, which sits near the largest
//    entries; the window holds it unless the row's mass is spread over
//    values close to zero (then the radix passes take the row).
// The threshold and every value above it are usually inside; an entry above
// the window sends the row to k_filter's radix passes.  k_filter_win reads
// a row's thresholds from the counts instead of passes over the row.
constexpr int kWinKeys = 512;
constexpr int kWinPKeys = 1024;
constexpr int kWinSlot = 1024;         // counts kept per sweep block (the larger window)
constexpr int kWinTopMargin = 192;
constexpr int kWinPTopMargin = 256;
constexpr int kWinKBelow = 128;
constexpr int kWinLines = 8;           // runs of 64 entries sampled by each sweep block
constexpr uint32_t kWinMinKey = 0x80;  // just above the key of -inf (0x7F)

// Where the filtered sweep leaves its window (null pointers: no window).
struct WinArgs {
  const int32_t* top_k;  // [B] or null
  const float* top_p;    // [B] or null
  double* partd;         // [rows][nc]: top-p alone: each chunk's sum 2^(x c - fl(xmax c)) in float64
  uint16_t* whist;       // [rows][nblk][kWinSlot]: entries per window value, per sweep block
  uint32_t* wflag;       // [rows][nblk]: 1 when the block saw an entry above the window
  uint32_t* wwin;        // [rows]: the window, lowest key | highest key << 16
  uint32_t* fall;        // [rows]: rows k_filter_win leaves to the radix passes, nfall of them
  uint32_t* nfall;       // [1], cleared by the sweep
  int nblk;              // sweep blocks per row
};

// Shape of a draft tree (nodes in topological order, parent[i] < i), shared
// by the batch; passed by value as a kernel argument.
constexpr int kMaxTree = SV_MAX_K + 1;
// Each table starts on a 4-byte boundary of the kernel arguments, so a
// lookup with a wave-uniform index can be one scalar load of the word that
// holds the entry (an unaligned byte would be a vector load to wait for).
struct TreeShape {
  int n;                                   // nodes
  int n_int;                               // nodes with children
  alignas(4) int8_t kid_off[kMaxTree + 1]; // children of v: kids[kid_off[v] .. kid_off[v + 1])
  alignas(4) int8_t kids[kMaxTree];        // in increasing index order
  alignas(4) int8_t int_node[kMaxTree];    // node whose draft row is swept row n + i
  alignas(4) int8_t int_idx[kMaxTree];     // i for a node with children, -1 for a leaf
};

static_assert(offsetof(TreeShape, kid_off) % 4 == 0 && offsetof(TreeShape, kids) % 4 == 0 &&
                  offsetof(TreeShape, int_node) % 4 == 0 && offsetof(TreeShape, int_idx) % 4 == 0,
              "shape tables start on 4-byte boundaries");

// Entry i of a byte table of the kernel arguments, i wave-uniform: the
// 32-bit word that holds it, then the byte.
__device__ __forceinline__ int arg_byte(const int8_t* tab, int i) {
  const uint32_t w = reinterpret_cast<const uint32_t*>(tab)[i >> 2];
  return (int)(int8_t)(w >> ((i & 3) * 8));
}

// Where a tree walk stands between rounds.
struct TreeState {
  int v;          // current node
  int pos;        // position among v's children of the next one to test
  int n;          // accepted nodes so far
  int fin;        // the scheduled pass feeds the final draw
  double n_prev;  // residual mass at coef_prev (1: q itself)
};

// The rows one sequence sweeps, and the tokens recorded in each.  Chain:
// target rows 0..K, then draft rows 0..K-1; target and draft row j record
// drafted token j (index b K + j).
struct ChainRows {
  int K;
  __device__ __forceinline__ int count() const { return 2 * K + 1; }
  __device__ __forceinline__ bool valid(int, int) const { return true; }
  __device__ __forceinline__ bool is_draft(int j) const { return j > K; }
  __device__ __forceinline__ int n_target() const { return K + 1; }
  __device__ __forceinline__ size_t row(int b, int j) const {
    return j <= K ? (size_t)b * (K + 1) + j : (size_t)b * K + (j - K - 1);
  }
  template <class F>
  __device__ __forceinline__ void for_each_token(int b, int j, F&& f) const {
    const int jj = j <= K ? j : j - K - 1;
    if (jj < K) f((size_t)b * K + jj);
  }
};

// Tree: target rows of all nodes, then draft rows of the nodes with
// children; the rows of node v record the tokens of v's children (index
// b n + child).
struct TreeRows {
  TreeShape s;
  __device__ __forceinline__ int count() const { return s.n + s.n_int; }
  __device__ __forceinline__ bool valid(int, int) const { return true; }
  __device__ __forceinline__ bool is_draft(int j) const { return j >= s.n; }
  __device__ __forceinline__ int n_target() const { return s.n; }
  __device__ __forceinline__ int node(int j) const {
    return j < s.n ? j : arg_byte(s.int_node, j - s.n);
  }
  __device__ __forceinline__ size_t row(int b, int j) const { return (size_t)b * s.n + node(j); }
  template <class F>
  __device__ __forceinline__ void for_each_token(int b, int j, F&& f) const {
    const int v = node(j);
    for (int k = arg_byte(s.kid_off, v); k < arg_byte(s.kid_off, v + 1); ++k)
      f((size_t)b * s.n + arg_byte(s.kids, k));
  }
};

// A shape per sequence (shapes[b], built on the device): the same row order
// with room for N - 1 draft rows per sequence; the rows past a sequence's
// own count are not swept.  Lookups read the shape's words from memory (b
// and j are uniform in a workgroup: scalar loads).
struct TreeRowsSeq {
  const TreeShape* shapes;
  int N;
  __device__ __forceinline__ int count() const { return 2 * N - 1; }
  __device__ __forceinline__ bool valid(int b, int j) const { return j < N || j - N < shapes[b].n_int; }
  __device__ __forceinline__ bool is_draft(int j) const { return j >= N; }
  __device__ __forceinline__ int n_target() const { return N; }
  __device__ __forceinline__ int node(int b, int j) const {
    return j < N ? j : arg_byte(shapes[b].int_node, j - N);
  }
  __device__ __forceinline__ size_t row(int b, int j) const { return (size_t)b * N + node(b, j); }
  template <class F>
  __device__ __forceinline__ void for_each_token(int b, int j, F&& f) const {
    const TreeShape& s = shapes[b];
    const int v = node(b, j);
    for (int k = arg_byte(s.kid_off, v); k < arg_byte(s.kid_off, v + 1); ++k)
      f((size_t)b * N + arg_byte(s.kids, k));
  }
};

// Per-chunk float64 sums (e = unnormalised weight in the 2^((x - xmax) c) frame).
struct ChunkSums {
  double eq, ep;  // sum of e_q, e_p over the chunk
  double a, b;    // the same sums over the entries with q > p
};

// The same sums per 256-entry sub-chunk; the final draw narrows
// chunk -> sub-chunk -> entry.
constexpr int kSub = 256;
constexpr int kSubPerChunk = kResChunk / kSub;
struct SubSums {
  double a, b, q, p;
};

// ---- Hand-offs between workgroups of one kernel (the chain's draw and the
// tree's rounds: the workgroup that completes a sequence's pass takes the
// next step).  The sums one workgroup leaves for another are stored with
// device-scope relaxed atomic stores, which write through the XCD's L2, and
// read with device-scope relaxed atomic loads, which do not return a stale
// L2 copy; the writer drains its memory counter before it counts itself in,
// and the reader reads only after it has seen the count complete.  No
// device-scope fence is used: on this chip a release fence writes back and an
// acquire fence invalidates the whole L2 of the XCD.
typedef unsigned long long u64;

__device__ __forceinline__ double ld_agent_d(const double* p) {
  return __longlong_as_double((long long)__hip_atomic_load(
      reinterpret_cast<const u64*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void st_agent_d(double* p, double v) {
  __hip_atomic_store(reinterpret_cast<u64*>(p), (u64)__double_as_longlong(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
// Every memory access this wave has issued is complete (its device-scope
// stores are visible to every workgroup).
__device__ __forceinline__ void vm_drain() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);          // vmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
__device__ __forceinline__ double ld_sum(const double* p, bool agent) {
  return agent ? ld_agent_d(p) : *p;
}
__device__ __forceinline__ SubSums ld_sub_sums(const SubSums* p) {
  const double* d = reinterpret_cast<const double*>(p);
  return SubSums{ld_agent_d(d), ld_agent_d(d + 1), ld_agent_d(d + 2), ld_agent_d(d + 3)};
}
__device__ __forceinline__ ChunkSums ld_chunk_sums(const ChunkSums* p, bool agent) {
  if (!agent) return *p;
  const double* d = reinterpret_cast<const double*>(p);
  return ChunkSums{ld_agent_d(d), ld_agent_d(d + 1), ld_agent_d(d + 2), ld_agent_d(d + 3)};
}

__host__ __device__ inline int sweep_chunks(int V) { return (V + kSweepChunk - 1) / kSweepChunk; }
__host__ __device__ inline int res_chunks(int V) { return (V + kResChunk - 1) / kResChunk; }

__device__ __forceinline__ float temp_of(const float* temp, int b, int force_greedy) {
  return force_greedy ? 0.f : temp[b];
}

// Load VN logits at [e, e + VN) of a row, -inf past V.
template <typename T, bool kAligned, bool kNT = false>
__device__ __forceinline__ void load_vec(const T* __restrict__ row, int e, int V,
                                         float (&x)[Vec16<T>::N]) {
  constexpr int VN = Vec16<T>::N;
  if (kAligned) {
    if (e < V) {
      if (kNT) Vec16<T>::load_nt(row + e, x);
      else Vec16<T>::load(row + e, x);
    } else {
#pragma unroll
      for (int k = 0; k < VN; ++k) x[k] = -INFINITY;
    }
  } else {
#pragma unroll
    for (int k = 0; k < VN; ++k) x[k] = (e + k < V) ? Vec16<T>::one(row + e + k) : -INFINITY;
  }
}

// Raw 16-byte vector of a row at entry e (a multiple of the vector width),
// read without a branch: past V the load goes to the row start and the
// result is replaced by -inf bit patterns, so the loads of a lane can all be
// in flight at once.
template <typename T>
__device__ __forceinline__ u32x4_t past_end_neg_inf(const u32x4_t r, bool in) {
  constexpr unsigned kNegInf = sizeof(T) == 2 ? 0xFF80FF80u : 0xFF800000u;
  return in ? r : u32x4_t{kNegInf, kNegInf, kNegInf, kNegInf};
}
__device__ __forceinline__ u32x4_t and_raw(const u32x4_t a, const u32x4_t b) {
  return u32x4_t{a.x & b.x, a.y & b.y, a.z & b.z, a.w & b.w};
}
template <typename T>
__device__ __forceinline__ u32x4_t load_clamped(const T* __restrict__ row, int e, int V) {
  return *reinterpret_cast<const u32x4_t*>(row + (e < V ? e : 0));
}
template <typename T>
__device__ __forceinline__ u32x4_t load_raw(const T* __restrict__ row, int e, int V) {
  return past_end_neg_inf<T>(load_clamped<T>(row, e, V), e < V);
}

template <typename T>
__device__ __forceinline__ void widen_raw(const u32x4_t r, float (&f)[Vec16<T>::N]) {
  if constexpr (sizeof(T) == 2) {
    Vec16<uint16_t>::widen(r, f);
  } else {
    f[0] = __uint_as_float(r.x); f[1] = __uint_as_float(r.y);
    f[2] = __uint_as_float(r.z); f[3] = __uint_as_float(r.w);
  }
}

// Element loads for rows that are not 16-byte aligned, repacked as raw
// vectors (exact: the values are logits of type T or -inf).
template <typename T>
__device__ __forceinline__ u32x4_t load_raw_unaligned(const T* __restrict__ row, int e, int V) {
  float x[Vec16<T>::N];
  load_vec<T, false>(row, e, V, x);
  if constexpr (sizeof(T) == 2) {
    unsigned w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = (__float_as_uint(x[2 * k]) >> 16) | (__float_as_uint(x[2 * k + 1]) & 0xffff0000u);
    return u32x4_t{w[0], w[1], w[2], w[3]};
  } else {
    return u32x4_t{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                   __float_as_uint(x[3])};
  }
}

// The logits of the tokens a swept row tests, for the accept tests: each
// written by the lane that holds it (xd[2 token + is_draft]).
template <typename T, class Rows>
__device__ __forceinline__ void record_draft_logits(const Rows& rows, int b, int j, int chunk,
                                                    int lane, bool is_draft, int V,
                                                    const float (&x)[kSweepChunk / (64 * Vec16<T>::N)][Vec16<T>::N],
                                                    const int32_t* __restrict__ dtok,
                                                    float* __restrict__ xd) {
  constexpr int VN = Vec16<T>::N;
  constexpr int IT = kSweepChunk / (64 * VN);
  rows.for_each_token(b, j, [&](size_t ti) {
    const int dd = clampi(dtok[ti], 0, V - 1);
    const int off = dd - chunk * kSweepChunk;
    if (off >= 0 && off < kSweepChunk && lane == (off / VN) % 64) {
      const int it_d = off / (64 * VN), k_d = off % VN;
      float v = 0.f;
#pragma unroll
      for (int it = 0; it < IT; ++it)
#pragma unroll
        for (int k = 0; k < VN; ++k)
          if (it == it_d && k == k_d) v = x[it][k];
      xd[ti * 2 + (is_draft ? 1 : 0)] = v;
    }
  });
}

// The top-k window (see kWinKeys) from the maximum sm of the row's sample:
// lowest key | highest key << 16.
__device__ __forceinline__ uint32_t topk_window(float sm, int tk, int V) {
  const uint32_t ksm = key32_of(sm) >> 16;
  const uint32_t ktop = min(ksm + (uint32_t)kWinTopMargin, 0xFFFFu);
  const uint32_t wide = ktop >= kWinMinKey + (kWinKeys - 1) ? ktop - (kWinKeys - 1) : kWinMinKey;
  const uint32_t near = ksm >= kWinMinKey + kWinKBelow ? ksm - kWinKBelow : kWinMinKey;
  const uint32_t kbase = (long long)tk * 256 <= (long long)V ? max(near, wide) : wide;
  return kbase | (ktop << 16);
}

// The top-p window (see kWinPKeys) from the maximum sm of the row's sample:
// lowest key | highest key << 16.
__device__ __forceinline__ uint32_t topp_window(float sm) {
  const uint32_t ksm = key32_of(sm) >> 16;
  const uint32_t ktop = min(ksm + (uint32_t)kWinPTopMargin, 0xFFFFu);
  const uint32_t kbase = ktop >= kWinMinKey + (kWinPKeys - 1) ? ktop - (kWinPKeys - 1) : kWinMinKey;
  return kbase | ((kbase + (kWinPKeys - 1)) << 16);
}

// Vector index of sampled vector i of a row of nvec vectors: runs of 8
// vectors (64 bf16 entries, one 128-byte line), nruns of them spread evenly.
__device__ __forceinline__ int sample_vec(int i, int nruns, int nvec) {
  return min((int)(((long long)(i >> 3) * nvec) / nruns) + (i & 7), nvec - 1);
}

// One block of the sweep of a filtered bf16 row (16-byte aligned): each
// chunk's raw maximum, and the count of every value of the row's window
// (see kWinKeys) among the block's entries.  A filtered row's law is
// normalised over its kept set, so the decision takes the kept mass from
// k_filter instead of the sweep's sum: only top-p alone sums masses here (its
// target needs the row's whole mass), in the chunk's own frame, in fp32 per
// vector of 8 and float64 beyond (partd; part.y gets the chunk's sum).  An
// entry above the window sets the block's flag: k_filter then takes its
// radix passes for the row.  All four waves reach both barriers (a wave past
// the row's last chunk only takes part in the counts' write-out).
template <class Rows>
__device__ __forceinline__ void sweep_window_block(const uint16_t* __restrict__ src, const Rows& rows,
                                                   int b, int j, int row, bool is_draft, float t,
                                                   int tk, bool k_on, int V, int nc,
                                                   const int32_t* __restrict__ dtok,
                                                   float2* __restrict__ part, float* __restrict__ xd,
                                                   const WinArgs& wa) {
  constexpr int VN = Vec16<uint16_t>::N;
  constexpr int IT = kSweepChunk / (64 * VN);
  static_assert(kWinSlot == 4 * kThreads && kWinKeys == 2 * kThreads, "window values per thread");
  static_assert(kWinLines * 8 == 64, "one sampled vector per lane");
  __shared__ uint32_t s_hist[kWinSlot + 64];       // + one spare bin per lane
  __shared__ uint32_t s_flag;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int chunk = blockIdx.y * 4 + wave;
  const bool live = chunk < nc;
  const int base = chunk * kSweepChunk + lane * VN;
  const bool full = (chunk + 1) * kSweepChunk <= V;
  // The window from this block's read of the sample runs, requested ahead
  // of the chunk's rows, so it is ready while they are still arriving.
  float xs[VN];
  Vec16<uint16_t>::load(src + (size_t)sample_vec(lane, kWinLines, V / VN) * VN, xs);
  float x[IT][VN];
  if (live) {
    if (full) {
#pragma unroll
      for (int it = 0; it < IT; ++it) Vec16<uint16_t>::load_nt(src + base + it * 64 * VN, x[it]);
    } else {
#pragma unroll
      for (int it = 0; it < IT; ++it) load_vec<uint16_t, true, true>(src, base + it * 64 * VN, V, x[it]);
    }
  }
#pragma unroll
  for (int i = 0; i < kWinSlot / kThreads; ++i) s_hist[tid + i * kThreads] = 0u;
  if (tid == 0) s_flag = 0u;
  float sm = xs[0];
#pragma unroll
  for (int k = 1; k < VN; ++k) sm = fmaxf(sm, xs[k]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sm = fmaxf(sm, __shfl_xor(sm, off, 64));
  const uint32_t win = k_on ? topk_window(sm, tk, V) : topp_window(sm);
  const uint32_t kbase = win & 0xFFFFu, ktop = win >> 16;
  if (live) record_draft_logits<uint16_t>(rows, b, j, chunk, lane, is_draft, V, x, dtok, xd);
  float flo, fhi;
  key_bounds(kbase << 16, (ktop << 16) | 0xFFFFu, flo, fhi);
  __syncthreads();                                 // counts cleared
  if (live) {
    float xm = -INFINITY;
#pragma unroll
    for (int it = 0; it < IT; ++it)
#pragma unroll
      for (int k = 0; k < VN; ++k) xm = fmaxf(xm, x[it][k]);
    float xw = xm;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) xw = fmaxf(xw, __shfl_xor(xw, off, 64));
    // An entry above the window sends the row to the radix passes.
    if (__ballot(xm > fhi) && lane == 0) atomicOr(&s_flag, 1u);
    if (kbase > 0x8000u) {
      // A window of positive values above +0 (the usual case): the bin from
      // the raw bits without a branch, bf16 bits - lowest bits as an unsigned
      // (negative values and values outside the window give more than the
      // window holds), capped at the lane's spare bin.
      const uint32_t kb = kbase - 0x8000u;
#pragma unroll
      for (int it = 0; it < IT; ++it)
#pragma unroll
        for (int k = 0; k < VN; ++k) {
          const uint32_t d = (__float_as_uint(x[it][k]) >> 16) - kb;
          atomicAdd(&s_hist[min(d, (uint32_t)(kWinSlot + lane))], 1u);
        }
    } else {
#pragma unroll
      for (int it = 0; it < IT; ++it)
#pragma unroll
        for (int k = 0; k < VN; ++k) {
          const float v = x[it][k];
          if (v >= flo && v <= fhi) atomicAdd(&s_hist[(key32_of(v) >> 16) - kbase], 1u);
        }
    }
    double sd = 0.0;
    if (!k_on && xw != -INFINITY) {
      // Top-p alone: masses 2^(x c - fl(xw c)) (entries past V are -inf: 0).
      const float c = kLog2e / t;
      const float m = xw * c;
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        float vs = 0.f;
#pragma unroll
        for (int k = 0; k < VN; ++k) vs += exp2_dev(__builtin_fmaf(x[it][k], c, -m));
        sd += (double)vs;
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) sd += __shfl_xor(sd, off, 64);
    }
    if (lane == 0) {
      part[(size_t)row * nc + chunk] = make_float2(xw, (float)sd);
      if (!k_on) wa.partd[(size_t)row * nc + chunk] = sd;
    }
  }
  __syncthreads();                                 // every entry counted
  // A block holds at most 4 kSweepChunk = 16384 entries: counts fit 16 bits.
  const size_t hb = ((size_t)row * wa.nblk + blockIdx.y) * kWinSlot;
  if (k_on) {
    const int i0 = 2 * tid;
    *reinterpret_cast<uint32_t*>(wa.whist + hb + i0) = s_hist[i0] | (s_hist[i0 + 1] << 16);
  } else {
    const int i0 = 4 * tid;
    *reinterpret_cast<uint2*>(wa.whist + hb + i0) =
        make_uint2(s_hist[i0] | (s_hist[i0 + 1] << 16), s_hist[i0 + 2] | (s_hist[i0 + 3] << 16));
  }
  if (tid == 0) {
    wa.wflag[(size_t)row * wa.nblk + blockIdx.y] = s_flag;
    if (blockIdx.y == 0) wa.wwin[row] = win;
  }
}

// ---------------------------------------------------------------------------
// k_sweep: grid (B * rows.count(), ceil(nc / 4)); block 256 = 4 waves, one
// chunk each.  part[row * nc + chunk] = (raw max, sum 2^(x c - fl(max c)))
// or, greedy, (max value, argmax index bits).  Also zeroes pcnt[0..B).
// kWin: rows with a filter (bf16, aligned) also count their window
// (sweep_window_block).
// ---------------------------------------------------------------------------
template <typename T, bool kAligned, class Rows, bool kWin = false>
__global__ __launch_bounds__(kThreads) void k_sweep(
    const T* __restrict__ tgt, const T* __restrict__ drf, const int32_t* __restrict__ dtok,
    const float* __restrict__ temp, Rows rows, int B, int V, int nc, int force_greedy,
    float2* __restrict__ part, float* __restrict__ xd, unsigned* __restrict__ pcnt, WinArgs wa) {
  // Clears the per-sequence pass counts the later kernels count in with (and
  // the filter's fallback list).
  if (blockIdx.y == 0 && (int)blockIdx.x < B && threadIdx.x == 0) pcnt[blockIdx.x] = 0u;
  if (kWin && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *wa.nfall = 0u;
  const int R = rows.count();
  // Every sequence's target rows first, then the draft rows: a greedy
  // sequence's draft-row workgroups leave at once, and in this order they are
  // dispatched after all the rows that are read.
  const int NT = rows.n_target(), ND = R - NT;
  const int r = blockIdx.x;
  const int b = r < B * NT ? r / NT : (r - B * NT) / ND;
  const int j = r < B * NT ? r - b * NT : NT + (r - B * NT) - b * ND;
  const int row = b * R + j;                   // row index of the statistics
  const bool is_draft = rows.is_draft(j);
  // Greedy sequences never read draft rows, so a draft row waits for its
  // sequence's temperature; a target row is read whatever it is, and its
  // loads are issued before the temperature arrives.
  if (is_draft && !(temp_of(temp, b, force_greedy) > 0.f)) return;
  if (!rows.valid(b, j)) return;                 // a per-sequence shape with fewer rows
  const T* src = (is_draft ? drf : tgt) + rows.row(b, j) * (size_t)V;
  if constexpr (kWin && kAligned && sizeof(T) == 2) {
    const float tw = temp_of(temp, b, force_greedy);
    const int tk = wa.top_k ? wa.top_k[b] : 0;
    const float tp = wa.top_p ? wa.top_p[b] : 1.f;
    const bool k_on = tk > 0 && tk < V, p_on = tp > 0.f && tp < 1.f;
    if (tw > 0.f && (k_on || p_on)) {              // block-uniform
      sweep_window_block<Rows>(src, rows, b, j, row, is_draft, tw, tk, k_on, V, nc, dtok, part, xd, wa);
      return;
    }
  }
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int chunk = blockIdx.y * 4 + wave;
  if (chunk >= nc) return;
  constexpr int VN = Vec16<T>::N;
  constexpr int IT = kSweepChunk / (64 * VN);
  const int base = chunk * kSweepChunk + lane * VN;
  // Every chunk but a row's last lies wholly inside the vocabulary: that
  // (wave-uniform) case needs no per-entry range checks.
  const bool full = kAligned && (chunk + 1) * kSweepChunk <= V;
  float x[IT][VN];
  if (full) {
#pragma unroll
    for (int it = 0; it < IT; ++it) Vec16<T>::load_nt(src + base + it * 64 * VN, x[it]);
  } else {
#pragma unroll
    for (int it = 0; it < IT; ++it) load_vec<T, kAligned, true>(src, base + it * 64 * VN, V, x[it]);
  }
  const float t = temp_of(temp, b, force_greedy);
  const bool greedy = !(t > 0.f);
  if (!greedy) record_draft_logits<T>(rows, b, j, chunk, lane, is_draft, V, x, dtok, xd);
  float2 res;
  if (greedy) {
    float mv = -INFINITY;
    int mi = INT32_MAX;
    if (full) {
      // Entries visited in increasing index: strict > keeps the lowest index.
      mv = x[0][0];
      mi = base;
#pragma unroll
      for (int it = 0; it < IT; ++it)
#pragma unroll
        for (int k = 0; k < VN; ++k)
          if (x[it][k] > mv) { mv = x[it][k]; mi = base + it * 64 * VN + k; }
    } else {
#pragma unroll
      for (int it = 0; it < IT; ++it)
#pragma unroll
        for (int k = 0; k < VN; ++k) {
          const int e = base + it * 64 * VN + k;
          if (e < V && (x[it][k] > mv || mi == INT32_MAX)) { mv = x[it][k]; mi = e; }
        }
    }
    wave_am_reduce(mv, mi);
    res = make_float2(mv, __int_as_float(mi));
  } else {
    const float c = kLog2e / t;
    float xm = -INFINITY;
#pragma unroll
    for (int it = 0; it < IT; ++it)
#pragma unroll
      for (int k = 0; k < VN; ++k) xm = fmaxf(xm, x[it][k]);
    // Lane statistics relative to the lane's scaled max, then a butterfly
    // merge of (scaled max, sum) pairs; the raw max rides along.
    float m = xm * c;
    float s = 0.f;
    if (xm != -INFINITY) {
#pragma unroll
      for (int it = 0; it < IT; ++it)
#pragma unroll
        for (int k = 0; k < VN; ++k) s += exp2_dev(__builtin_fmaf(x[it][k], c, -m));
    }
    wave_ms_reduce(m, s);
    float xr = xm;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) xr = fmaxf(xr, __shfl_xor(xr, off, 64));
    // The merged m equals fl(xr * c): scaling is monotone, so the largest
    // scaled lane max is the scaled largest raw max.
    res = make_float2(xr, s);
  }
  if (lane == 0) part[(size_t)row * nc + chunk] = res;
}

// Merge of the nc chunk statistics of one row by a group of 16 lanes (one
// DPP row), fixed order: lane j takes chunks j, j + 16, ... in order, then the
// group combines by DPP moves (xor 1, xor 2, mirror in 8, mirror in 16).
// Sampling rows give (raw max, sum relative to fl(raw max * c)); greedy rows
// (max value, lowest argmax).
// Each step is a symmetric merge, so both lanes of a pairing, and in the end
// all 16 lanes, hold the same values.
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, true));
}

template <int kCtrl>
__device__ __forceinline__ void group16_step(bool greedy, float& x, float& y, float& xr) {
  const float x2 = dpp_f<kCtrl>(x), y2 = dpp_f<kCtrl>(y), xr2 = dpp_f<kCtrl>(xr);
  if (greedy) {
    int i = __float_as_int(y);
    am_merge(x, i, x2, __float_as_int(y2));
    y = __int_as_float(i);
  } else {
    ms_merge(x, y, x2, y2);
    xr = fmaxf(xr, xr2);
  }
}

__device__ __forceinline__ void merge_row16(const float2* __restrict__ pr, int nc, bool greedy, float c,
                                            int j, float& a, float& bb) {
  float x = -INFINITY, y = greedy ? __int_as_float(INT32_MAX) : 0.f, xr = -INFINITY;
  auto take = [&](const float2 p) {
    if (greedy) {
      int i = __float_as_int(y);
      am_merge(x, i, p.x, __float_as_int(p.y));
      y = __int_as_float(i);
    } else {
      ms_merge(x, y, p.x * c, p.y);
      xr = fmaxf(xr, p.x);
    }
  };
  // The first four chunks of the lane are requested together (clamped
  // indices, the duplicates not merged), then merged in order: one round
  // trip for rows of up to 64 chunks (V <= 2^18 at 4096 per chunk).
  constexpr int kPre = 4;
  float2 pp[kPre];
#pragma unroll
  for (int u = 0; u < kPre; ++u) pp[u] = pr[min(j + 16 * u, nc - 1)];
#pragma unroll
  for (int u = 0; u < kPre; ++u)
    if (j + 16 * u < nc) take(pp[u]);
  for (int k = j + 16 * kPre; k < nc; k += 16) take(pr[k]);
  group16_step<0xB1>(greedy, x, y, xr);     // quad_perm [1,0,3,2]
  group16_step<0x4E>(greedy, x, y, xr);     // quad_perm [2,3,0,1]
  group16_step<0x141>(greedy, x, y, xr);    // row_half_mirror
  group16_step<0x140>(greedy, x, y, xr);    // row_mirror
  a = greedy ? x : xr;
  bb = y;
}

// Write the K+1 output slots (threads 0..K of the block), the accepted count
// and the committed length (thread 0).  The drafted tokens come from `sd`.
__device__ __forceinline__ void emit(int b, int K, int n, int tok, const int* __restrict__ sd,
                                     int32_t* __restrict__ out, int32_t* __restrict__ nacc,
                                     int32_t* __restrict__ kv_len, unsigned long long* counters) {
  const int i = threadIdx.x;
  if (i <= K) out[(size_t)b * (K + 1) + i] = (i < n) ? sd[i] : (i == n ? tok : -1);
  if (i == 0) {
    nacc[b] = n;
    kv_len[b] = kv_len[b] + n + 1;
    if (counters) {
      atomicAdd(&counters[0], (unsigned long long)K);
      atomicAdd(&counters[1], (unsigned long long)n);
    }
  }
}

// emit() for a thread that holds its own draft token (thread i < K: d_{i+1}).
__device__ __forceinline__ void emit_own(int b, int K, int n, int tok, int my_draw,
                                         int32_t* __restrict__ out, int32_t* __restrict__ nacc,
                                         int32_t* __restrict__ kv_len, unsigned long long* counters) {
  const int i = threadIdx.x;
  if (i <= K) out[(size_t)b * (K + 1) + i] = (i < n) ? my_draw : (i == n ? tok : -1);
  if (i == 0) {
    nacc[b] = n;
    kv_len[b] = kv_len[b] + n + 1;
    if (counters) {
      atomicAdd(&counters[0], (unsigned long long)K);
      atomicAdd(&counters[1], (unsigned long long)n);
    }
  }
}

// ---------------------------------------------------------------------------
// k_filter: grid (B * rows.count()), block 512 (two per CU): the top-k / top-p thresholds
// of one row (the sweep's row set and order) by radix selection over its order keys,
// most significant digit first:
// 12 bits, then 4 (bf16) or 12 and 8 (fp32).  Each pass histograms the
// entries that match the digits chosen so far into up to 4096 bins of counts
// (top-k) or masses (top-p), and the block picks the bin where the running
// total from the top reaches the target.  The first pass takes every entry
// (no branch around its adds); later passes test membership with two float
// compares against the value range of the chosen bin, and only members
// compute a key.  The wide first digit splits each exponent's entries over
// 16 bins, so fewer threads add to the same bin at once.  For bf16 the last
// pass works on single values: counts only, each bin's mass being its count
// times the value's weight.  Masses are 2^(x c - fl(xmax c)) in fp32, added
// as 40-bit fixed point with integer atomics: the sums do not depend on the
// order of the adds (bitwise reproducible) and are exact to ~1e-7 of the
// row's mass.
// ---------------------------------------------------------------------------
constexpr int kFilterThreads = 512;
constexpr int kFilterWaves = kFilterThreads / 64;
constexpr int kFilterBins = 4096;
static_assert(kFilterBins % kFilterThreads == 0, "whole bins per thread in filter_pick");
constexpr double kFix = 1099511627776.0;          // 2^40
constexpr int kWinBins = 16;                      // 12-bit bins whose single values a first pass counts

// 16-byte vectors per batch of a thread (two batches are in registers at
// once); half as many where each load is several (rows that do not start on
// a 16-byte boundary).
template <typename T, bool kAligned>
constexpr int filter_batch() { return kAligned ? 4 : 2; }

// fp32 rows: three digits of the 32-bit key, 12, 12 and 8 bits, most
// significant first (a bf16 row takes 12 bits, then its 16 single values).
constexpr int kF32Levels = 3;
__device__ __forceinline__ int f32_digit_bits(int level) { return level == 2 ? 8 : 12; }

// floor(2^40 w) as an integer, for 0 <= w < 2^24: t = 256 w is exact, its
// integer part gives the high word and its fraction times 2^32 (exact,
// truncated by the conversion) the low word (weights below 2^-40 give 0).
__device__ __forceinline__ unsigned long long fixed40(float w) {
  const float t = w * 256.0f;
  const uint32_t hi = (uint32_t)t;
  const uint32_t lo = (uint32_t)(__builtin_amdgcn_fractf(t) * 4294967296.0f);
  return ((unsigned long long)hi << 32) | lo;
}

// Streams a row through f(x, e): x the VN widened logits of the vector at
// entry e (past V: -inf).  Each thread alternates between two named batches
// of filter_batch vectors, requesting the next batch before it uses the
// current one (no register copy between them, so no wait for the batch just
// requested).
template <typename T, bool kAligned, class F>
__device__ __forceinline__ void filter_scan(const T* __restrict__ row, int V, F&& f) {
  constexpr int VN = Vec16<T>::N;
  constexpr int NB = filter_batch<T, kAligned>();
  constexpr int kStep = kFilterThreads * VN * NB;
  auto fetch = [&](u32x4_t (&r)[NB], int base) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int e = base + j * kFilterThreads * VN;
      r[j] = kAligned ? load_raw<T>(row, e, V) : load_raw_unaligned<T>(row, e, V);
    }
  };
  auto use = [&](const u32x4_t (&r)[NB], int base) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      float x[VN];
      widen_raw<T>(r[j], x);
      f(x, base + j * kFilterThreads * VN);
    }
  };
  int base = threadIdx.x * VN;
  if (base >= V) return;
  u32x4_t ra[NB], rb[NB];
  fetch(ra, base);
  for (; base < V; base += 2 * kStep) {
    if (base + kStep < V) fetch(rb, base + kStep);
    use(ra, base);
    if (base + kStep >= V) break;
    if (base + 2 * kStep < V) fetch(ra, base + 2 * kStep);
    use(rb, base + kStep);
  }
}

// One pass over a row: each entry with flo <= x <= fhi (every entry when
// kAll) adds to bin (key32 >> shift) & (2^width - 1) of h: 1 (top-k) or its
// weight 2^(x c - mc) in 40-bit fixed point (top-p).  Each thread requests
// filter_batch vectors before it uses any; with kAll the adds are not
// branched around (entries past V add 0).
// Extra counts of a bf16 first pass (12-bit digit): with kWin the single
// values of the kWinBins bins from wlo (hx [kWinBins][16], the value's index
// being the low 4 bits of its 16-bit key, as in the last pass), with kBinMass
// also the masses of the counted entries per bin (hm [4096]).
struct FirstPassExtra {
  uint32_t wlo;
  unsigned long long* hx;
  unsigned long long* hm;
};

template <typename T, bool kAligned, bool kMass, bool kAll, bool kWin = false,
          bool kBinMass = false>
__device__ __forceinline__ void filter_hist(const T* __restrict__ row, int V, float c, float mc,
                                            float flo, float fhi, int shift, int width,
                                            unsigned long long* h,
                                            const FirstPassExtra& ex = FirstPassExtra{0u, nullptr, nullptr}) {
  constexpr int VN = Vec16<T>::N;
  for (int i = threadIdx.x; i < kFilterBins; i += kFilterThreads) {
    h[i] = 0ull;
    if (kBinMass) ex.hm[i] = 0ull;
  }
  if (kWin)
    for (int i = threadIdx.x; i < kWinBins * 16; i += kFilterThreads) ex.hx[i] = 0ull;
  __syncthreads();
  // The single-value count of an entry with key `key` in bin `bin`.
  auto count_value = [&](uint32_t key, uint32_t bin) {
    const uint32_t d = bin - ex.wlo;
    if (d < (uint32_t)kWinBins) atomicAdd(&ex.hx[d * 16 + __builtin_amdgcn_ubfe(key, 16, 4)], 1ull);
  };
  filter_scan<T, kAligned>(row, V, [&](const float (&x)[VN], int e) {
#pragma unroll
    for (int k = 0; k < VN; ++k) {
      const bool inb = kAligned ? e < V : e + k < V;
      if (kAll) {
        const uint32_t key = key32_of(x[k]);
        const uint32_t bin = __builtin_amdgcn_ubfe(key, shift, width);
        unsigned long long v;
        if (kMass) v = fixed40(exp2_dev(__builtin_fmaf(x[k], c, -mc)));
        else v = 1ull;
        atomicAdd(&h[bin], inb ? v : 0ull);
        if (kWin && inb) count_value(key, bin);
      } else if (inb && x[k] >= flo && x[k] <= fhi) {
        const uint32_t key = key32_of(x[k]);
        const uint32_t bin = __builtin_amdgcn_ubfe(key, shift, width);
        if (kMass || kBinMass) {
          const unsigned long long w = fixed40(exp2_dev(__builtin_fmaf(x[k], c, -mc)));
          if (kMass) atomicAdd(&h[bin], w);
          else atomicAdd(&h[bin], 1ull);
          if (kBinMass) atomicAdd(&ex.hm[bin], w);
        } else {
          atomicAdd(&h[bin], 1ull);
        }
        if (kWin) count_value(key, bin);
      }
    }
  });
  __syncthreads();
}

// bf16 rows, last pass: inside the chosen 12-bit bin (flo <= x <= fhi) each
// of the 16 bins is one bf16 value, so counts suffice: the mass of a bin is
// its count times the value's weight, the same integer as the sum of the
// entries' weights.  bin = low 4 bits of the value's key, i.e. of the bf16
// bits, complemented for negative values (flip = 15).  With kAbove each
// thread also sums the weights of the entries above the bin (x > fhi).
template <bool kAligned, bool kAbove>
__device__ __forceinline__ unsigned long long filter_hist_exact(const uint16_t* __restrict__ row,
                                                                int V, float c, float mc,
                                                                float flo, float fhi, uint32_t flip,
                                                                unsigned long long* h) {
  constexpr int VN = Vec16<uint16_t>::N;
  if (threadIdx.x < 16) h[threadIdx.x] = 0ull;
  __syncthreads();
  unsigned long long above = 0ull;
  filter_scan<uint16_t, kAligned>(row, V, [&](const float (&x)[VN], int e) {
#pragma unroll
    for (int k = 0; k < VN; ++k) {
      const bool inb = kAligned ? e < V : e + k < V;
      if (inb && x[k] >= flo && x[k] <= fhi)
        atomicAdd(&h[__builtin_amdgcn_ubfe(__float_as_uint(x[k]), 16, 4) ^ flip], 1ull);
      if (kAbove && inb && x[k] > fhi) above += fixed40(exp2_dev(__builtin_fmaf(x[k], c, -mc)));
    }
  });
  __syncthreads();
  return above;
}

// The bf16 value with 16-bit key k, widened.
__device__ __forceinline__ float key16_value(uint32_t k) {
  const uint32_t hb = (k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu);
  return __uint_as_float(hb << 16);
}

// Block sum of one integer per thread (exact in any order).
__device__ __forceinline__ unsigned long long block_sum_u64(unsigned long long v,
                                                            unsigned long long* s_red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  __syncthreads();
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  unsigned long long tot = 0ull;
#pragma unroll
  for (int w = 0; w < kFilterWaves; ++w) tot += s_red[w];
  __syncthreads();
  return tot;
}

// The block picks the largest bin whose running total from the top, plus
// the total `above` carried from the higher digits, reaches `target`; it
// adds the totals of the bins above the pick to `above`.  If no bin reaches
// (only by rounding), the lowest nonempty bin.  Thread t holds bins
// P t .. P t + P - 1, P = kFilterBins / kFilterThreads.  All threads return
// the same values.
__device__ __forceinline__ int filter_pick(const unsigned long long* h, int nbins, double target,
                                           unsigned long long& above, unsigned long long* s_w,
                                           int* s_pick, unsigned long long* s_above) {
  constexpr int P = kFilterBins / kFilterThreads;   // bins per thread
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b0 = P * tid;
  unsigned long long v[P], loc = 0ull;
#pragma unroll
  for (int k = 0; k < P; ++k) {
    v[k] = (b0 + k < nbins) ? h[b0 + k] : 0ull;
    loc += v[k];
  }
  // Inclusive suffix sums over the lanes of a wave (lanes l..63), then over
  // the waves above.
  unsigned long long suf = loc;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned long long t = __shfl_down(suf, off, 64);
    if (lane + off < 64) suf += t;
  }
  if (lane == 0) s_w[wave] = suf;                  // the wave's total
  __syncthreads();
  unsigned long long wabove = 0ull;
  for (int w = wave + 1; w < kFilterWaves; ++w) wabove += s_w[w];
  unsigned long long acc = above + wabove + (suf - loc);   // everything above this thread's bins
  int hit = -1, nonempty = 1 << 30;
#pragma unroll
  for (int k = P - 1; k >= 0; --k) {
    acc += v[k];
    if (hit < 0 && (double)acc >= target) hit = b0 + k;
    if (v[k]) nonempty = b0 + k;
  }
  // Block max of hit, block min of nonempty.
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    hit = max(hit, __shfl_xor(hit, off, 64));
    nonempty = min(nonempty, __shfl_xor(nonempty, off, 64));
  }
  if (lane == 0) { s_pick[wave] = hit; s_pick[kFilterWaves + wave] = nonempty; }
  __syncthreads();
  int sel = -1, ne = 1 << 30;
  for (int w = 0; w < kFilterWaves; ++w) { sel = max(sel, s_pick[w]); ne = min(ne, s_pick[kFilterWaves + w]); }
  if (sel < 0) sel = ne < nbins ? ne : 0;
  // The owner of bin sel knows the total above it.
  if (tid == sel / P) {
    unsigned long long ab = above + wabove + (suf - loc);
#pragma unroll
    for (int k = P - 1; k >= 0; --k)
      if (b0 + k > sel) ab += v[k];
    *s_above = ab;
  }
  __syncthreads();
  above = *s_above;
  __syncthreads();
  return sel;
}

// A lower bound for the k-th largest key of a row, for k no larger than the
// number of threads that read an entry: each thread takes the largest entry
// of one vector of a sample spread evenly over the row, and the block counts
// those maxima in the 4096 bins of their top 12 key bits.  The bin where the
// count from the top reaches k starts at a key that at least k maxima (so at
// least k entries) reach.  The sample is 1/16 of a bf16 row at the llama
// vocabulary; the selection passes that follow then only see the entries at
// or above the bound (a few per thousand for small k).
template <typename T, bool kAligned>
__device__ __forceinline__ uint32_t topk_bound(const T* __restrict__ row, int V, int tk,
                                               unsigned long long* h, unsigned long long* s_w,
                                               int* s_pick, unsigned long long* s_above) {
  constexpr int VN = Vec16<T>::N;
  const int nvec = (V + VN - 1) / VN;              // vectors in the row
  const int nt = min(kFilterThreads, nvec);        // threads that read one
  float mx = -INFINITY;
  if ((int)threadIdx.x < nt) {
    const int e = (int)(((long long)threadIdx.x * nvec / nt)) * VN;
    const u32x4_t raw = kAligned ? load_raw<T>(row, e, V) : load_raw_unaligned<T>(row, e, V);
    float x[VN];
    widen_raw<T>(raw, x);
#pragma unroll
    for (int k = 0; k < VN; ++k)
      if (kAligned || e + k < V) mx = fmaxf(mx, x[k]);
  }
  for (int i = threadIdx.x; i < kFilterBins; i += kFilterThreads) h[i] = 0ull;
  __syncthreads();
  if ((int)threadIdx.x < nt) atomicAdd(&h[key32_of(mx) >> 20], 1ull);
  __syncthreads();
  unsigned long long above = 0ull;
  const int sel = filter_pick(h, kFilterBins, (double)tk, above, s_w, s_pick, s_above);
  return (uint32_t)sel << 20;
}

// The mass of the entries with x >= flo, in 40-bit fixed point: per-thread
// sums, then a block sum (integers: exact in any order).
template <typename T, bool kAligned>
__device__ __forceinline__ unsigned long long filter_kept_mass(const T* __restrict__ row, int V,
                                                               float c, float mc, float flo,
                                                               unsigned long long* s_red) {
  constexpr int VN = Vec16<T>::N;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  unsigned long long acc = 0ull;
  filter_scan<T, kAligned>(row, V, [&](const float (&x)[VN], int e) {
#pragma unroll
    for (int k = 0; k < VN; ++k) {
      const bool inb = kAligned ? e < V : e + k < V;
      if (inb && x[k] >= flo) acc += fixed40(exp2_dev(__builtin_fmaf(x[k], c, -mc)));
    }
  });
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  __syncthreads();
  if (lane == 0) s_red[wave] = acc;
  __syncthreads();
  unsigned long long tot = 0ull;
#pragma unroll
  for (int w = 0; w < kFilterWaves; ++w) tot += s_red[w];
  __syncthreads();
  return tot;
}

// The largest of a wave's 64 N bins (lane l holds bins N l .. N l + N - 1)
// whose running total from the top reaches target; -1 when none does.
// ab_out: the running total above the bin, vs_out the bin's own value (both
// the same in every lane).  The order of the integer adds does not matter.
template <int N>
__device__ __forceinline__ int wave_pick(const unsigned long long (&v)[N], double target, int lane,
                                         unsigned long long& ab_out, unsigned long long& vs_out) {
  unsigned long long loc = 0ull;
#pragma unroll
  for (int k = 0; k < N; ++k) loc += v[k];
  unsigned long long suf = loc;                    // lanes l .. 63
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned long long t = __shfl_down(suf, off, 64);
    if (lane + off < 64) suf += t;
  }
  unsigned long long acc = suf - loc;
  int hit = -1;
  unsigned long long ab = 0ull, vs = 0ull;
#pragma unroll
  for (int k = N - 1; k >= 0; --k) {
    if (hit < 0 && (double)(acc + v[k]) >= target) {
      hit = N * lane + k;
      ab = acc;
      vs = v[k];
    }
    acc += v[k];
  }
  int h = hit;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) h = max(h, __shfl_xor(h, off, 64));
  if (h < 0) return -1;
  const int owner = __builtin_amdgcn_readfirstlane(h / N);
  auto bcast = [&](unsigned long long x) {
    return ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)(x >> 32), owner) << 32) |
           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, owner);
  };
  ab_out = bcast(ab);
  vs_out = bcast(vs);
  return h;
}

// The thresholds of one row from its window of 64 N values (one wave; see
// k_filter_win): writes the RowFilter and returns true, or false when the
// window does not decide the row.
template <int N>
__device__ __forceinline__ bool window_thresholds(int row, int nc, float c, float mc, int tk, float tp,
                                                  bool k_on, bool p_on, uint32_t kbase,
                                                  const float2* __restrict__ part, const WinArgs& wa,
                                                  RowFilter* __restrict__ filt, int lane) {
  // Every load first: the blocks' flags and counts and, for top-p alone, the
  // chunk sums (after the caller's chunk maxima).
  bool bad = false;
  for (int y = lane; y < wa.nblk; y += 64) bad = bad || wa.wflag[(size_t)row * wa.nblk + y] != 0u;
  uint32_t cnt[N];
#pragma unroll
  for (int k = 0; k < N; ++k) cnt[k] = 0u;
  const uint16_t* hp = wa.whist + (size_t)row * wa.nblk * kWinSlot + N * lane;
  for (int y0 = 0; y0 < wa.nblk; y0 += 8) {
    uint4 v[8][N / 8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int h = 0; h < N / 8; ++h)
        v[q][h] = y0 + q < wa.nblk
                      ? *reinterpret_cast<const uint4*>(hp + (size_t)(y0 + q) * kWinSlot + 8 * h)
                      : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int h = 0; h < N / 8; ++h) {
        const uint32_t w4[4] = {v[q][h].x, v[q][h].y, v[q][h].z, v[q][h].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          cnt[8 * h + 2 * k] += w4[k] & 0xFFFFu;
          cnt[8 * h + 2 * k + 1] += w4[k] >> 16;
        }
      }
  }
  double z = 0.0;
  if (p_on && !k_on) {
    // The row's mass in its frame: chunk sums in chunk order per lane, then
    // a fixed-order wave sum.
    for (int k = lane; k < nc; k += 64) {
      const size_t i = (size_t)row * nc + k;
      const float mk = part[i].x * c;             // the chunk's frame, as the sweep took it
      z += wa.partd[i] * exp2((double)mk - (double)mc);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off, 64);
  }
  if (__ballot(bad)) return false;
  unsigned long long v[N], ab = 0ull, vs = 0ull;
  int sel = 0;
  if (k_on) {
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] = cnt[k];
    sel = wave_pick<N>(v, (double)tk, lane, ab, vs);
    if (sel < 0) return false;                     // fewer than k entries in the window
  }
  // Masses of the values from the top-k threshold up (all of the window
  // without top-k).
  unsigned long long loc = 0ull;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const int i = N * lane + k;
    const float xv = key16_value(kbase + (uint32_t)i);
    v[k] = i >= sel ? cnt[k] * fixed40(exp2_dev(__builtin_fmaf(xv, c, -mc))) : 0ull;
    loc += v[k];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) loc += __shfl_xor(loc, off, 64);
  unsigned long long kept = loc;                   // the set's mass
  if (p_on) {
    const double target = k_on ? (double)tp * (double)loc : (double)tp * z * kFix;
    if ((double)loc < target) return false;        // the threshold lies under the window
    sel = wave_pick<N>(v, target, lane, ab, vs);
    if (sel < 0) return false;
    kept = ab + vs;
  }
  if (lane == 0) filt[row] = RowFilter{kbase + (uint32_t)sel, 0u, (double)kept / kFix};
  return true;
}

// k_filter_win: grid (B * rows.count()), one wave per row: the thresholds of
// a row the filtered sweep counted in a window, from the sweep blocks'
// counts.  Summed per window value, the counts from the top give the top-k
// threshold (the largest value with at least k entries at or above it); a
// value's mass is its count times its weight, the same integer as the sum of
// its entries' weights in the radix passes, and the masses from the top give
// the top-p threshold and the kept mass.  Top-p alone takes the row's mass
// from the sweep's float64 chunk sums, moved into the row's frame.  Rows
// without a filter get the empty RowFilter.  A row the window does not decide
// (an entry above the window, fewer than k entries in it, or a top-p target
// not reached at its lowest value) goes on the list k_filter, launched next,
// takes through the radix passes.
template <class Rows>
__global__ __launch_bounds__(64) void k_filter_win(
    const float* __restrict__ temp, const int32_t* __restrict__ top_k, const float* __restrict__ top_p,
    Rows rows, int V, int nc, int force_greedy, const float2* __restrict__ part,
    RowFilter* __restrict__ filt, WinArgs wa) {
  static_assert(kWinKeys == 8 * 64 && kWinPKeys == 16 * 64, "8 or 16 window values per lane");
  const int R = rows.count();
  const int row = blockIdx.x;
  const int b = row / R;
  const int j = row - b * R;
  const int lane = threadIdx.x;
  if (!rows.valid(b, j)) return;
  const float t = temp_of(temp, b, force_greedy);
  const int tk = top_k ? top_k[b] : 0;
  const float tp = top_p ? top_p[b] : 1.f;
  const bool k_on = tk > 0 && tk < V;
  const bool p_on = tp > 0.f && tp < 1.f;
  if (!(t > 0.f) || (!k_on && !p_on)) {
    if (lane == 0) filt[row] = RowFilter{0u, 0u, 0.0};
    return;
  }
  const float c = kLog2e / t;
  const uint32_t kbase = wa.wwin[row] & 0xFFFFu;
  float xr = -INFINITY;
  for (int k = lane; k < nc; k += 64) xr = fmaxf(xr, part[(size_t)row * nc + k].x);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) xr = fmaxf(xr, __shfl_xor(xr, off, 64));
  const float mc = xr * c;
  const bool done = k_on ? window_thresholds<8>(row, nc, c, mc, tk, tp, k_on, p_on, kbase, part, wa, filt, lane)
                         : window_thresholds<16>(row, nc, c, mc, tk, tp, k_on, p_on, kbase, part, wa, filt, lane);
  if (!done && lane == 0) wa.fall[atomicAdd(wa.nfall, 1u)] = (uint32_t)row;
}

// The radix selection of one row (k_filter).
template <typename T, bool kAligned, class Rows>
__device__ __forceinline__ void filter_row(int row, const T* __restrict__ tgt, const T* __restrict__ drf,
                                           const float* __restrict__ temp,
                                           const int32_t* __restrict__ top_k,
                                           const float* __restrict__ top_p, const Rows& rows, int V,
                                           int nc, int force_greedy, const float2* __restrict__ part,
                                           RowFilter* __restrict__ filt) {
  __shared__ unsigned long long h[kFilterBins];
  __shared__ unsigned long long s_w[kFilterWaves];
  __shared__ int s_pick[2 * kFilterWaves];
  __shared__ unsigned long long s_above;
  __shared__ unsigned long long s_wt[16];
  __shared__ unsigned long long hx[kWinBins * 16];   // single values of the window's bins
  __shared__ unsigned long long hm[kFilterBins];      // top-k alone: masses per first-digit bin
  __shared__ float s_xr;
  const int R = rows.count();
  const int b = row / R;
  const int j = row - b * R;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (!rows.valid(b, j)) return;                 // a per-sequence shape with fewer rows
  const float t = temp_of(temp, b, force_greedy);
  const int tk = top_k ? top_k[b] : 0;
  const float tp = top_p ? top_p[b] : 1.f;
  const bool k_on = tk > 0 && tk < V;
  const bool p_on = tp > 0.f && tp < 1.f;
  if (!(t > 0.f) || (!k_on && !p_on)) {
    if (tid == 0) filt[row] = RowFilter{0u, 0u, 0.0};
    return;
  }
  const T* src = (rows.is_draft(j) ? drf : tgt) + rows.row(b, j) * (size_t)V;
  const float c = kLog2e / t;
  // The row's raw maximum, merged from the sweep's chunk maxima as the decision does.
  if (wave == 0) {
    float xr = -INFINITY;
    for (int k = lane; k < nc; k += 64) xr = fmaxf(xr, part[(size_t)row * nc + k].x);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) xr = fmaxf(xr, __shfl_xor(xr, off, 64));
    if (lane == 0) s_xr = xr;
  }
  __syncthreads();
  const float mc = s_xr * c;
  // Keys are handled in the 32-bit space of the widened floats; a bf16 key
  // is the top 16 bits, so its passes stop at bit 16.
  constexpr int kStop = sizeof(T) == 2 ? 16 : 0;
  uint32_t lo = 0u;                                // 32-bit keys below this are filtered out
  unsigned long long kept_mass = 0ull;
  bool have_mass = false;
  // Small k: restrict the top-k passes to the entries at or above a bound
  // (each of min(512, vectors in the row) threads contributes one vector's
  // maximum, so the count from the top reaches k).
  if (k_on && tk <= min(kFilterThreads, (V + Vec16<T>::N - 1) / Vec16<T>::N))
    lo = topk_bound<T, kAligned>(src, V, tk, h, s_w, s_pick, &s_above);
  for (int f = 0; f < 2; ++f) {
    const bool by_mass = (f == 1);
    if (by_mass ? !p_on : !k_on) continue;
    uint32_t prefix = 0u;
    unsigned long long above = 0ull;
    double target = by_mass ? 0.0 : (double)tk;
    if constexpr (sizeof(T) == 2) {
      // bf16: the 12-bit first digit, then the chosen bin's single values.
      // When the first pass only sees the entries at or above a bound (top-k
      // with its sampled bound, top-p over the top-k set) it also counts the
      // single values of the kWinBins bins from the bound's bin, and a chosen
      // bin among them needs no second pass.  (Over every entry, top-p alone,
      // those extra counts cost about as much as the pass they save.)
      const bool need_above = !by_mass && !p_on;
      const bool windowed = lo != 0u;
      const uint32_t wlo = min(lo >> 20, (uint32_t)(kFilterBins - kWinBins));
      const FirstPassExtra ex{wlo, hx, hm};
      if (lo == 0u) {
        if (by_mass) filter_hist<T, kAligned, true, true>(src, V, c, mc, 0.f, 0.f, 20, 12, h);
        else filter_hist<T, kAligned, false, true>(src, V, c, mc, 0.f, 0.f, 20, 12, h);
      } else {
        float flo, fhi;
        key_bounds(lo, 0xFFFFFFFFu, flo, fhi);
        if (by_mass) filter_hist<T, kAligned, true, false, true>(src, V, c, mc, flo, fhi, 20, 12, h, ex);
        else if (need_above)
          filter_hist<T, kAligned, false, false, true, true>(src, V, c, mc, flo, fhi, 20, 12, h, ex);
        else filter_hist<T, kAligned, false, false, true>(src, V, c, mc, flo, fhi, 20, 12, h, ex);
      }
      if (by_mass) {
        // The kept set's mass (all of the row, or its top-k set) sets the target.
        unsigned long long part_sum = 0ull;
        for (int i = tid; i < kFilterBins; i += kFilterThreads) part_sum += h[i];
        target = (double)tp * (double)block_sum_u64(part_sum, s_w);
      }
      const int sel0 = filter_pick(h, kFilterBins, target, above, s_w, s_pick, &s_above);
      prefix = (uint32_t)sel0;
      // The 16 single values of bin sel0 into h[0..15]: from the window, or
      // by one more pass.
      unsigned long long ab = 0ull;            // top-k alone: mass above bin sel0
      if (windowed && (uint32_t)sel0 - wlo < (uint32_t)kWinBins) {
        if (need_above) {
          unsigned long long part_ab = 0ull;
          for (int i = tid; i < kFilterBins; i += kFilterThreads)
            if (i > sel0) part_ab += hm[i];
          ab = block_sum_u64(part_ab, s_w);
        }
        if (tid < 16) h[tid] = hx[(sel0 - wlo) * 16 + tid];
        __syncthreads();
      } else {
        float flo, fhi;
        key_bounds(max(prefix << 20, lo), (uint32_t)((((unsigned long long)prefix + 1) << 20) - 1),
                   flo, fhi);
        const uint32_t flip = (prefix & 0x800u) ? 0u : 15u;
        if (need_above) {
          ab = filter_hist_exact<kAligned, true>(src, V, c, mc, flo, fhi, flip, h);
          ab = block_sum_u64(ab, s_w);
        } else {
          filter_hist_exact<kAligned, false>(src, V, c, mc, flo, fhi, flip, h);
        }
      }
      if (tid < 16) {
        const float xv = key16_value((prefix << 4) | (uint32_t)tid);
        const unsigned long long w = fixed40(exp2_dev(__builtin_fmaf(xv, c, -mc)));
        if (by_mass) h[tid] *= w;
        else s_wt[tid] = w;
      }
      __syncthreads();
      const int sel = filter_pick(h, 16, target, above, s_w, s_pick, &s_above);
      prefix = (prefix << 4) | (uint32_t)sel;
      if (by_mass) {
        kept_mass = above + h[sel];
      } else if (need_above) {
        // Top-k alone: the mass of the kept set, {x > bin} plus the values
        // of the bin from sel up.
        unsigned long long m = ab;
        for (int i = sel; i < 16; ++i) m += h[i] * s_wt[i];
        kept_mass = m;
        have_mass = true;
      }
      __syncthreads();
      lo = prefix << kStop;                        // the k-th largest key, or the top-p key
      have_mass = have_mass || by_mass;
      continue;
    }
    // fp32: three range passes.
    int shift = 32;
    for (int lv = 0; lv < kF32Levels; ++lv) {
      const int width = f32_digit_bits(lv);
      const int high = shift;                      // the bits above `high` are fixed: prefix
      shift -= width;
      if (lv == 0 && lo == 0u) {
        if (by_mass) filter_hist<T, kAligned, true, true>(src, V, c, mc, 0.f, 0.f, shift, width, h);
        else filter_hist<T, kAligned, false, true>(src, V, c, mc, 0.f, 0.f, shift, width, h);
      } else {
        const uint32_t klo = high >= 32 ? 0u : prefix << high;
        const uint32_t khi = high >= 32 ? 0xFFFFFFFFu
                                        : (uint32_t)((((unsigned long long)prefix + 1) << high) - 1);
        float flo, fhi;
        key_bounds(max(klo, lo), khi, flo, fhi);
        if (by_mass) filter_hist<T, kAligned, true, false>(src, V, c, mc, flo, fhi, shift, width, h);
        else filter_hist<T, kAligned, false, false>(src, V, c, mc, flo, fhi, shift, width, h);
      }
      if (by_mass && lv == 0) {
        // The kept set's mass (all of the row, or its top-k set) sets the target.
        unsigned long long part_sum = 0ull;
        for (int i = tid; i < kFilterBins; i += kFilterThreads) part_sum += h[i];
        target = (double)tp * (double)block_sum_u64(part_sum, s_w);
      }
      const int sel = filter_pick(h, 1 << width, target, above, s_w, s_pick, &s_above);
      prefix = (prefix << width) | (uint32_t)sel;
      if (by_mass && shift == kStop) kept_mass = above + h[sel];
      __syncthreads();
    }
    lo = prefix << kStop;                          // the k-th largest key, or the top-p key
    have_mass = have_mass || by_mass;
  }
  // Top-k alone: the kept set's mass in one more pass (top-p's passes give it).
  if (!have_mass) {
    float flo, fhi;
    key_bounds(lo, 0xFFFFFFFFu, flo, fhi);
    kept_mass = filter_kept_mass<T, kAligned>(src, V, c, mc, flo, s_w);
  }
  if (tid == 0) filt[row] = RowFilter{lo >> kStop, 0u, (double)kept_mass / kFix};
}

// Without a window: one block per row (grid B * rows.count()).
template <typename T, bool kAligned, class Rows>
__global__ __launch_bounds__(kFilterThreads, 4) void k_filter(
    const T* __restrict__ tgt, const T* __restrict__ drf, const float* __restrict__ temp,
    const int32_t* __restrict__ top_k, const float* __restrict__ top_p, Rows rows, int V, int nc,
    int force_greedy, const float2* __restrict__ part, RowFilter* __restrict__ filt) {
  filter_row<T, kAligned, Rows>(blockIdx.x, tgt, drf, temp, top_k, top_p, rows, V, nc, force_greedy,
                                part, filt);
}

// After k_filter_win: a grid of any size takes the rows on its list (a
// kernel of its own: the loop's live values would spill k_filter's
// registers).
template <typename T, bool kAligned, class Rows>
__global__ __launch_bounds__(kFilterThreads, 4) void k_filter_list(
    const T* __restrict__ tgt, const T* __restrict__ drf, const float* __restrict__ temp,
    const int32_t* __restrict__ top_k, const float* __restrict__ top_p, Rows rows, int V, int nc,
    int force_greedy, const float2* __restrict__ part, RowFilter* __restrict__ filt, WinArgs wa) {
  const uint32_t n = *wa.nfall;
  for (uint32_t i = blockIdx.x; i < n; i += gridDim.x) {
    filter_row<T, kAligned, Rows>((int)wa.fall[i], tgt, drf, temp, top_k, top_p, rows, V, nc,
                                  force_greedy, part, filt);
    __syncthreads();                               // the block's LDS is reused for the next row
  }
}

// ---------------------------------------------------------------------------
// The chain's decision for sequence b (a block of NTH threads): merges the
// sweep's chunk statistics of its rows (one wave per row, fixed order), runs
// the K accept tests on K lanes at once (q/p in the log domain, float64),
// takes the first rejection by ballot and describes the pass that follows.
// Every thread gets the decision.  With `outputs`, a greedy sequence is also
// emitted and committed here, and the decision is stored to dec[b] for the
// final draw.
// ---------------------------------------------------------------------------
template <int NTH>
__device__ Decision decide_chain(int b, const int32_t* __restrict__ dtok, const float* __restrict__ uni,
                                 float t, int K, int V, int nc, const float2* __restrict__ part,
                                 const float* __restrict__ xd, const RowFilter* __restrict__ filt,
                                 int key16, bool outputs, Decision* __restrict__ dec,
                                 int32_t* __restrict__ out, int32_t* __restrict__ nacc,
                                 int32_t* __restrict__ kv_len, unsigned long long* counters) {
  __shared__ float s_a[kMaxRows], s_b[kMaxRows];
  __shared__ uint32_t s_kmin[kMaxRows];
  __shared__ float s_xq[SV_MAX_K], s_xp[SV_MAX_K], s_u[SV_MAX_K];
  __shared__ int s_d[SV_MAX_K], s_draw[SV_MAX_K];
  __shared__ int s_n;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int R = 2 * K + 1;
  const bool greedy = !(t > 0.f);
  const int rows = greedy ? K + 1 : R;
  const float c = greedy ? 0.f : kLog2e / t;
  // All loads are independent: the drafted tokens, their logits (recorded
  // by the sweep), the uniforms, the filters and the row statistics.
  const float2* pb = part + (size_t)b * R * nc;
  int draw = 0;
  float xq = 0.f, xp = 0.f, uu = 0.f;
  if (tid < K) {
    draw = dtok[(size_t)b * K + tid];
    if (!greedy) {
      xq = xd[((size_t)b * K + tid) * 2];
      xp = xd[((size_t)b * K + tid) * 2 + 1];
      uu = uni[(size_t)b * (K + 1) + tid];
    }
  }
  // Row statistics: 16 lanes per row, NTH / 16 rows at a time.
  for (int r0 = 0; r0 < rows; r0 += NTH / 16) {
    const int r = r0 + (tid >> 4);
    const bool head = (tid & 15) == 0 && r < rows;
    // A filtered row: its law is renormalised over the kept set.
    const RowFilter rf = (filt && !greedy && head) ? filt[(size_t)b * R + r] : RowFilter{0u, 0u, 0.0};
    float a, bb;
    merge_row16(pb + (size_t)min(r, rows - 1) * nc, nc, greedy, c, tid & 15, a, bb);
    if (head) {
      s_a[r] = a;
      s_b[r] = rf.key_min ? (float)rf.mass : bb;
      s_kmin[r] = rf.key_min;
    }
  }
  if (tid < K) {
    s_draw[tid] = draw;
    s_d[tid] = clampi(draw, 0, V - 1);
    s_xq[tid] = xq;
    s_xp[tid] = xp;
    s_u[tid] = uu;
  }
  __syncthreads();
  // Accept tests of all K drafts at once (lanes of wave 0), then the first
  // rejection.
  if (wave == 0) {
    bool acc = false;
    if (lane < K) {
      const int i = lane;
      if (greedy) {
        acc = (s_d[i] == __float_as_int(s_b[i]));
      } else if (s_xp[i] == -INFINITY || float_key(s_xp[i], key16) < s_kmin[K + 1 + i]) {
        acc = true;                                   // p(d) == 0 (filtered out included)
      } else if (float_key(s_xq[i], key16) < s_kmin[i]) {
        acc = false;                                  // q(d) == 0: filtered out of the target
      } else {
        // q/p = 2^((xq c - mq) - (xp c - mp)) * sp / sq with m = fl(xmax c),
        // taken in the log domain so small probabilities do not underflow.
        const double mq = (double)(s_a[i] * c), mp = (double)(s_a[K + 1 + i] * c);
        const double ly = ((double)s_xq[i] * (double)c - mq) - ((double)s_xp[i] * (double)c - mp);
        const double r = exp2(ly) * ((double)s_b[K + 1 + i] / (double)s_b[i]);
        acc = (double)s_u[i] < fmin(1.0, r);
      }
    }
    const unsigned long long rej = __ballot(lane < K && !acc);
    if (lane == 0) s_n = rej ? (int)__builtin_ctzll(rej) : K;
  }
  __syncthreads();
  const int n = s_n;
  if (greedy) {
    const Decision dd{kModeNone, n, 0, 0, 0.f, 0.f, 0.0, 0.0, 0.0};
    if (outputs) {
      if (tid == 0) dec[b] = dd;
      emit(b, K, n, __float_as_int(s_b[n]), s_draw, out, nacc, kv_len, counters);
    }
    return dd;
  }
  // One wave forms the decision (its float64 exp2 / log2 would cost every
  // wave of every block the same VALU time) and hands it over through LDS.
  __shared__ Decision s_dec;
  if (wave == 0) {
    const double cd = kLog2eD / (double)t;
    Decision dd{n < K ? kModeResid : kModeQ, n, b * (K + 1) + n, n < K ? b * K + n : 0,
                s_a[n], n < K ? s_a[K + 1 + n] : 0.f, 0.0, 1.0, 0.0, s_kmin[n],
                n < K ? s_kmin[K + 1 + n] : 0u};
    if (n < K) {
      // The sweep's normalisers, moved from the fl(xmax c) frame to the
      // 2^((x - xmax) c) frame of the exact pass.
      const double sq = (double)s_b[n] * exp2((double)(dd.xmq * c) - (double)dd.xmq * cd);
      const double sp = (double)s_b[K + 1 + n] * exp2((double)(dd.xmp * c) - (double)dd.xmp * cd);
      dd.theta = log2(sq) - log2(sp);
    }
    if (lane == 0) {
      s_dec = dd;
      if (outputs) dec[b] = dd;
    }
  }
  __syncthreads();
  return s_dec;
}

// Float64 2^a for a <= 0 (a slightly above 0 is fine too), to a relative
// error below 2e-13.  With k = round(256 a) (taken with the 2^52 + 2^51
// shifter, whose low word then holds k), 2^a = 2^floor(k/256) *
// 2^((k mod 256)/256) * 2^r, where r = a - k/256 is exact and |r| <= 1/512.
// The middle factor comes from a 256-entry table the block fills with the
// device's float64 exp2; 2^r is the Taylor series of e^(r ln 2) to degree 3
// (first dropped term (r ln 2)^4 / 24 < 1.4e-13); the power of two is applied
// exactly by ldexp.  Arguments are clamped at -1100, where ldexp underflows
// to exactly 0, so -inf weighs 0.  The final draw needs the weights to ~1e-10
// of the total mass at most, so 2e-13 leaves a wide margin.
//
// Callers pass A = 256 a, computed as x (256 c) - 256 fl(xmax c): scaling by
// 256 is exact, so A is exactly 256 times the unscaled exponent, the
// round(256 a) step becomes a plain add of the shifter, and the polynomial
// takes R = 256 r with its coefficients scaled by 2^-8n (also exact): every
// intermediate is the unscaled one times a power of two.  Split in two steps
// so a caller can issue the table reads of several entries before it needs
// any of them.
constexpr int kExpTable = 256;

struct Exp2Arg {
  double r;   // 256 a - k
  int k;      // round(256 a)
};

__device__ __forceinline__ Exp2Arg exp2_reduce(double A) {
  const double ac = fmax(A, -1100.0 * 256);
  const double shifter = 6755399441055744.0;               // 2^52 + 2^51
  const double t = ac + shifter;                           // shifter + k
  Exp2Arg e;
  e.k = __double2loint(t);
  e.r = ac - (t - shifter);                                // exact
  return e;
}

__device__ __forceinline__ double exp2_finish(const Exp2Arg& e, double tab_k) {
  double p = 3.3083026805413713e-09;                       // ln2^3 / 3! / 2^24
  p = fma(p, e.r, 3.6655655969101062e-06);                 // ln2^2 / 2! / 2^16
  p = fma(p, e.r, 2.7076061740622863e-03);                 // ln2 / 2^8
  p = fma(p, e.r, 1.0);
  return ldexp(tab_k * p, e.k >> 8);
}

__device__ __forceinline__ double exp2_neg(double A, const double* __restrict__ tab) {
  const Exp2Arg e = exp2_reduce(A);
  return exp2_finish(e, tab[e.k & (kExpTable - 1)]);
}

// Scaled exponent 256 (x - xmax) c of one entry, as x (256 c) - 256 fl(xmax c)
// (c256 = 256 c, xmc256 = 256 fl(xmax c), both exact): the rounding of
// fl(xmax c) is one factor common to the whole row, so it cancels in every
// normalised weight.
__device__ __forceinline__ double expo(float x, double c256, double xmc256) {
  return fma((double)x, c256, -xmc256);
}

// Float64 cross-lane steps for the sums and scans of the draw: DPP moves
// inside rows of 16 lanes and readlane across rows, a few cycles each where a
// generic shuffle goes through the LDS permute unit.  Each move takes the two
// halves of the double separately; lanes a move does not write read 0.
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kDppRowShr = 0x110;       // + n: row_shr:n
constexpr int kDppWaveShr1 = 0x138;     // wave_shr:1
constexpr int kDppRowMirror = 0x140;    // lane i <- 15 - i of its row
constexpr int kDppHalfMirror = 0x141;   // lane i <- 7 - i of its half row
constexpr int kDppBcast15 = 0x142;      // lane 15 of row r -> row r + 1
constexpr int kDppBcast31 = 0x143;      // lane 31 -> rows 2 and 3

template <int kCtrl, int kRowMask = 0xF, bool kBound = true>
__device__ __forceinline__ double dpp_d(double x) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(x), kCtrl, kRowMask, 0xF, kBound);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(x), kCtrl, kRowMask, 0xF, kBound);
  return __hiloint2double(hi, lo);
}

// Lane l's value in every lane (l wave-uniform).
__device__ __forceinline__ double readlane_d(double x, int l) {
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(x), l),
                          __builtin_amdgcn_readlane(__double2loint(x), l));
}

// Sum over each group of 8 lanes 8g..8g+7, in every lane of the group (fp
// addition is commutative, so both lanes of every pairing get the same value).
__device__ __forceinline__ double group8_sum_d(double x) {
  x += dpp_d<kDppXor1>(x);
  x += dpp_d<kDppXor2>(x);
  return x + dpp_d<kDppHalfMirror>(x);
}

// ---------------------------------------------------------------------------
// The final draw: narrows chunk -> sub-chunk (from the stored sums) -> entry
// (exact weights of one 256-entry run, one per thread), each level by an
// inclusive float64 scan in vocabulary order.
// ---------------------------------------------------------------------------
// What the draw's weights are: q, p, or (q - coef p)_+ (then isp = coef / sp).
enum : int { kDrawQ = 0, kDrawP = 1, kDrawResid = 2 };

__device__ __forceinline__ double chunk_mass(const ChunkSums& cs, int m, double isq, double isp) {
  return m == kDrawQ ? cs.eq * isq : (m == kDrawP ? cs.ep * isp : fmax(0.0, cs.a * isq - cs.b * isp));
}
__device__ __forceinline__ double sub_mass(const SubSums& ss, int m, double isq, double isp) {
  return m == kDrawQ ? ss.q * isq : (m == kDrawP ? ss.p * isp : fmax(0.0, ss.a * isq - ss.b * isp));
}

// Inclusive scan of one wave, in lane order: a scan inside each row of 16
// lanes, then the totals of the rows before.
__device__ __forceinline__ double wave_scan_d(double x) {
  x += dpp_d<kDppRowShr + 1>(x);
  x += dpp_d<kDppRowShr + 2>(x);
  x += dpp_d<kDppRowShr + 4>(x);
  x += dpp_d<kDppRowShr + 8>(x);
  x += dpp_d<kDppBcast15, 0xA, false>(x);     // rows 1 and 3
  x += dpp_d<kDppBcast31, 0xC, false>(x);     // rows 2 and 3
  return x;
}

// Sum of the wave, in every lane: row sums, then the four rows in a fixed
// order.
__device__ __forceinline__ double wave_sum_d(double x) {
  x = group8_sum_d(x);
  x += dpp_d<kDppRowMirror>(x);
  return (readlane_d(x, 0) + readlane_d(x, 16)) + (readlane_d(x, 32) + readlane_d(x, 48));
}

// One wave walks `cnt` masses (mass(i)) in order: returns the first index
// whose running sum from `base` exceeds `target` (or -1) and leaves in `base`
// the running sum before it; `lastpos` gets the last index of positive mass
// (-1 if none).
template <typename F>
__device__ __forceinline__ int wave_find(int cnt, F mass, double target, double& base, int& lastpos,
                                         int lane) {
  lastpos = -1;
  int found = -1;
  double carry = base;
  for (int s0 = 0; s0 < cnt; s0 += 64) {
    const int i = s0 + lane;
    const double m = i < cnt ? mass(i) : 0.0;
    const double incl = wave_scan_d(m) + carry;
    const unsigned long long pos = __ballot(m > 0.0);
    if (pos) lastpos = s0 + 63 - (int)__builtin_clzll(pos);
    const unsigned long long hit = __ballot(i < cnt && incl > target);
    if (found < 0 && hit) {
      const int l = (int)__builtin_ctzll(hit);
      found = s0 + l;
      base = (l == 0) ? carry : readlane_d(incl, l - 1);
    }
    carry = readlane_d(incl, 63);
  }
  return found;
}

// Sum of x over the first wave's lanes, chunk i on lane i % 64 (the one
// fixed order every caller uses).
template <typename F>
__device__ __forceinline__ double wave_chunk_sum(int ncr, F f, int lane) {
  double z = 0.0;
  for (int i = lane; i < ncr; i += 64) z += f(i);
  return wave_sum_d(z);
}

// The draw of one sequence (a block of kThreads threads) from the pass that
// decision d describes, given the pass's chunk sums cg [ncr] and sub-chunk
// sums sg [ncr][32], the exp table (filled here while the sums are loading
// when fill_table, else already filled) and the uniform u.  Returns the
// token in every thread, or -1 in every thread when d asks for no draw.
// d, u and t are first read after the sums are staged, so a caller can pass
// values whose loads are still in flight.
// kAgent: the sums were stored by other workgroups of the running kernel
// (device-scope loads, ncr <= 64): the first wave holds chunk i's sums on
// lane i, then the chosen chunk's sub-chunk sums, in registers; no staging.
template <typename T, bool kAgent = false>
__device__ __forceinline__ int locate_draw(const T* __restrict__ tgt, const T* __restrict__ drf,
                                           const Decision& d, float u, float t, int V, int ncr,
                                           const ChunkSums* __restrict__ cg,
                                           const SubSums* __restrict__ sg,
                                           double* __restrict__ s_exp, bool fill_table) {
  static_assert(kSub == kThreads, "one sub-chunk entry per thread");
  static_assert(kSubPerChunk <= 64, "one sub-chunk per lane");
  constexpr int kSubStage = kAgent ? 1 : 1024;   // sub-chunk sums staged in LDS (32 KB)
  __shared__ ChunkSums s_cs[kAgent ? 1 : kThreads];
  __shared__ SubSums s_ss[kSubStage];
  __shared__ double s_wtot[kThreads / 64];
  __shared__ int s_chunk, s_sub, s_fallback, s_mode, s_first, s_lastpos;
  __shared__ double s_base, s_target, s_isq, s_isp;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Chunk and sub-chunk sums staged in LDS together when they fit (V <= 2^18
  // for both, V <= 2^21 for the chunk sums), read in place otherwise: the
  // sub-chunk level then needs no second round trip to memory.  The loads
  // are issued before the table is filled and stored to LDS after it.
  const bool staged = !kAgent && ncr <= kThreads;
  const bool sub_staged = !kAgent && ncr * kSubPerChunk <= kSubStage;
  // Waves 0-1 stage the sums (all loads issued before any is stored), waves
  // 2-3 fill the table meanwhile.
  constexpr int kHalf = kThreads / 2;
  ChunkSums my_cs{};
  if constexpr (kAgent) {
    if (tid < min(ncr, 64)) my_cs = ld_chunk_sums(cg + tid, true);
    if (fill_table)
      for (int j = tid; j < kExpTable; j += kThreads) s_exp[j] = exp2((double)j * (1.0 / 256));
  } else if (tid < kHalf) {
    constexpr int kSubH = kSubStage / kHalf;
    static_assert(kThreads == 2 * kHalf, "two chunk sums per staging thread");
    // Clamped indices: every load and store is unconditional inside the
    // block-uniform branches (a clamped duplicate stores the same value to
    // the same slot), so the loads are all issued before the first store.
    // Sub-chunk sums that fit imply chunk sums that fit.
    const int c0 = min(tid, ncr - 1), c1 = min(tid + kHalf, ncr - 1);
    if (sub_staged) {
      const int nsub = ncr * kSubPerChunk;
      const ChunkSums r0 = cg[c0], r1 = cg[c1];
      SubSums rs[kSubH];
#pragma unroll
      for (int j = 0; j < kSubH; ++j) rs[j] = sg[min(tid + j * kHalf, nsub - 1)];
      __builtin_amdgcn_sched_barrier(0);
      s_cs[c0] = r0;
      s_cs[c1] = r1;
#pragma unroll
      for (int j = 0; j < kSubH; ++j) s_ss[min(tid + j * kHalf, nsub - 1)] = rs[j];
    } else if (staged) {
      const ChunkSums r0 = cg[c0], r1 = cg[c1];
      s_cs[c0] = r0;
      s_cs[c1] = r1;
    }
  } else if (fill_table) {
    for (int j = tid - kHalf; j < kExpTable; j += kHalf) s_exp[j] = exp2((double)j * (1.0 / 256));
  }
  __syncthreads();
  if (d.mode == kModeNone) return -1;                       // block-uniform
  const double cd = kLog2eD / (double)t;
  const T* trow = tgt + (size_t)d.trow * V;
  const T* drow = drf + (size_t)d.drow * V;
  const ChunkSums* cs = staged ? s_cs : cg;
  if (wave == 0) {
    // Chunk i's sums (every caller below asks only for i = lane + 64 j; with
    // kAgent only for i = lane).
    const auto chunk = [&](int i) { return kAgent ? my_cs : cs[i]; };
    // Exact normalisers, then the masses of the chunks.
    const double sq = wave_chunk_sum(ncr, [&](int i) { return chunk(i).eq; }, lane);
    const double sp = wave_chunk_sum(ncr, [&](int i) { return chunk(i).ep; }, lane);
    const double isq = 1.0 / sq;
    int m = d.mode == kModeQ ? kDrawQ : kDrawResid;
    double isp = m == kDrawQ ? 0.0 : d.coef / sp;
    double z = wave_chunk_sum(ncr, [&](int i) { return chunk_mass(chunk(i), m, isq, isp); }, lane);
    if (m == kDrawResid && !(z > 0.0)) {
      // Zero residual mass: the law stays (q - coef_prev p)_+ normalised, and
      // with no mass above p it equals p (q itself when coef_prev = 0).
      m = d.coef_prev == 0.0 ? kDrawQ : kDrawP;
      isp = 1.0 / sp;
      z = wave_chunk_sum(ncr, [&](int i) { return chunk_mass(chunk(i), m, isq, isp); }, lane);
    }
    const double target = (double)u * z;
    double base = 0.0;
    int lastpos;
    int ch = wave_find(ncr, [&](int i) { return chunk_mass(chunk(i), m, isq, isp); }, target, base,
                       lastpos, lane);
    int fb = 0;
    if (ch < 0) {                                             // rounding at u -> 1
      fb = 1;
      ch = lastpos < 0 ? 0 : lastpos;
    }
    // Sub-chunk level, same wave (no crossing is looked for once in fallback).
    const SubSums* ss = (sub_staged ? s_ss : sg) + (size_t)ch * kSubPerChunk;
    SubSums my_ss{};
    if (kAgent && lane < kSubPerChunk) my_ss = ld_sub_sums(ss + lane);
    double base2 = base;
    int lastsub;
    int sc = wave_find(kSubPerChunk,
                       [&](int j) { return sub_mass(kAgent ? my_ss : ss[j], m, isq, isp); },
                       fb ? (double)INFINITY : target, base2, lastsub, lane);
    if (sc < 0) {                                             // no crossing left: last positive run
      fb = 1;
      sc = lastsub < 0 ? 0 : lastsub;
    }
    if (lane == 0) {
      s_chunk = ch; s_sub = sc; s_fallback = fb; s_mode = m;
      s_base = base2; s_target = target; s_isq = isq; s_isp = isp;
      s_first = INT32_MAX; s_lastpos = -1;
    }
  }
  __syncthreads();
  const int ch = s_chunk;
  const int m = s_mode;
  const double isq = s_isq, isp = s_isp;
  const int e = ch * kResChunk + s_sub * kSub + tid;
  double w = 0.0;
  if (e < V) {
    const double c256 = cd * 256.0;
    float xq = m == kDrawP ? 0.f : Vec16<T>::one(trow + e);
    if (float_key(xq, sizeof(T) == 2) < d.kq) xq = -INFINITY;        // filtered out
    const double q = m == kDrawP ? 0.0
                                 : exp2_neg(expo(xq, c256, ((double)d.xmq * cd) * 256.0), s_exp) * isq;
    if (m == kDrawQ) {
      w = q;
    } else {
      float xp = Vec16<T>::one(drow + e);
      if (float_key(xp, sizeof(T) == 2) < d.kp) xp = -INFINITY;
      const double p = exp2_neg(expo(xp, c256, ((double)d.xmp * cd) * 256.0), s_exp) * isp;
      w = m == kDrawP ? p : fmax(0.0, q - p);
    }
  }
  // Inclusive prefix over the 256 entries in vocabulary order: a wave scan
  // plus the totals of the waves before (fixed order).
  const double incl = wave_scan_d(w);
  if (lane == 63) s_wtot[wave] = incl;
  __syncthreads();
  double run = s_base + incl;
  for (int ww = 0; ww < wave; ++ww) run += s_wtot[ww];
  if (!s_fallback && run > s_target) atomicMin(&s_first, e);
  if (w > 0.0) atomicMax(&s_lastpos, e);
  __syncthreads();
  int tok = s_first;
  if (tok == INT32_MAX) tok = s_lastpos;                     // no crossing: last positive weight
  if (tok < 0) tok = clampi(ch * kResChunk + s_sub * kSub, 0, V - 1);
  return tok;
}

// ---------------------------------------------------------------------------
// k_locate: grid (B); block 256.  The chain's final draw (sampling sequences
// only), then the outputs.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void k_locate(
    const T* __restrict__ tgt, const T* __restrict__ drf, const int32_t* __restrict__ dtok,
    const float* __restrict__ uni, const float* __restrict__ temp, int K, int V, int ncr,
    int force_greedy, const ChunkSums* __restrict__ csum, const SubSums* __restrict__ csub,
    const Decision* __restrict__ dec, int32_t* __restrict__ out, int32_t* __restrict__ nacc,
    int32_t* __restrict__ kv_len, unsigned long long* counters) {
  __shared__ double s_exp[kExpTable];
  const int b = blockIdx.x;
  // Every load is issued before any is waited for: the decision, the
  // temperature, the uniform and this thread's draft token fly while the
  // sums are staged (locate_draw reads them only after that, and returns -1
  // for sequences that need no draw).
  if (force_greedy) return;                     // every sequence greedy: nothing to draw
  const float t = temp[b];
  if (!(t > 0.f)) return;                       // greedy: emitted by the decision
  // Thread i < K emits draft i: it keeps its own token (no wait for it here).
  const int my_draw = (int)threadIdx.x < K ? dtok[(size_t)b * K + threadIdx.x] : 0;
  const float u = uni[(size_t)b * (K + 1) + K];
  const Decision d = dec[b];
  const int tok = locate_draw<T>(tgt, drf, d, u, t, V, ncr,
                                 csum + (size_t)b * ncr, csub + (size_t)b * ncr * kSubPerChunk, s_exp,
                                 true);
  if (tok < 0) return;
  emit_own(b, K, d.n, tok, my_draw, out, nacc, kv_len, counters);
}

// Filtered-out entries (order key below kmin) become -inf: weight 0, never
// classed q > c p.
template <typename T>
__device__ __forceinline__ void mask_row(float (&x)[Vec16<T>::N], uint32_t kmin) {
#pragma unroll
  for (int k = 0; k < Vec16<T>::N; ++k)
    x[k] = float_key(x[k], sizeof(T) == 2) < kmin ? -INFINITY : x[k];
}

// ---------------------------------------------------------------------------
// One block's share of the exact pass a decision asks for: chunk cr of the
// row pair, 8192 entries.
//
// Lane mapping: the 8 lanes of group g = lane / 8 in wave w own sub-chunk
// w * 8 + g (256 entries).  Each of their loads covers one 128-byte line of it,
// so an instruction of the wave still reads 8 whole lines, and a sub-chunk's
// sums need only 3 butterfly steps.
// ---------------------------------------------------------------------------
// kAgent: the sums are stored with device-scope stores, for a workgroup of
// the same kernel that reads them.  s_exp: the block's exp table (256
// doubles of LDS), filled here.
template <typename T, bool kAligned, bool kMask, bool kAgent = false>
__device__ __forceinline__ void residual_pass(const T* __restrict__ tgt, const T* __restrict__ drf,
                                              const Decision& d, float t, int V, int ncr, int b, int cr,
                                              ChunkSums* __restrict__ csum, SubSums* __restrict__ csub,
                                              double* __restrict__ s_exp) {
  constexpr int VN = Vec16<T>::N;
  constexpr int kLine = 8 * VN;                   // entries per 8-lane load (128 bytes)
  constexpr int IT = kSub / kLine;                // loads per lane per row
  static_assert(kThreads / 8 == kSubPerChunk, "one 8-lane group per sub-chunk");
  __shared__ SubSums s_sub[kSubPerChunk];
  const int tid = threadIdx.x;
  const int sub_i = tid >> 3, s = tid & 7;
  const bool bonus = d.mode == kModeQ;
  const double cd = kLog2eD / (double)t;
  const T* trow = tgt + (size_t)d.trow * (size_t)V;
  const T* drow = drf + (size_t)d.drow * (size_t)V;
  const int e0 = cr * kResChunk + sub_i * kSub + s * VN;
  // Loads first, so they are in flight while the table is filled, target and
  // draft vectors alternating so the first pair arrives first.  Aligned rows
  // set the vectors past V to -inf where they are used: a select right after
  // a load would wait for it there.
  u32x4_t rq[IT], rp[IT];
  if constexpr (kAligned) {
    // Without a branch: a bonus pass loads its target vectors twice (the
    // second load finds the line in flight, no extra HBM traffic) and uses
    // the AND of the two equal copies, so every load has a use on both paths
    // and stays here instead of being moved into one of them, and each
    // vector pair is waited for only where it is first used.
    const T* prow = bonus ? trow : drow;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      rq[i] = load_clamped<T>(trow, e0 + i * kLine, V);
      rp[i] = load_clamped<T>(prow, e0 + i * kLine, V);
    }
  } else {
#pragma unroll
    for (int i = 0; i < IT; ++i) rq[i] = load_raw_unaligned<T>(trow, e0 + i * kLine, V);
    if (!bonus) {
#pragma unroll
      for (int i = 0; i < IT; ++i) rp[i] = load_raw_unaligned<T>(drow, e0 + i * kLine, V);
    }
  }
  const auto vec = [&](const u32x4_t r, int i) {
    return kAligned ? past_end_neg_inf<T>(r, e0 + i * kLine < V) : r;
  };
  static_assert(kExpTable == kThreads, "one table entry per thread");
  s_exp[tid] = exp2((double)tid * (1.0 / 256));
  __syncthreads();
  // Exponents scaled by 256 (see exp2_reduce); all three scalings are exact.
  const double c256 = cd * 256.0;
  const double xmcq = ((double)d.xmq * cd) * 256.0, xmcp = ((double)d.xmp * cd) * 256.0;
  // Entries past V hold -inf: weight exactly 0, and never classed q > p.
  double sq = 0.0, sp = 0.0, sa = 0.0, sb = 0.0;
  // Per vector: reduce every exponent and issue all table reads, then the
  // polynomials (the reads' latency overlaps the reductions).
  if (bonus) {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      float xq[VN];
      widen_raw<T>(vec(kAligned ? and_raw(rq[i], rp[i]) : rq[i], i), xq);
      if (kMask) mask_row<T>(xq, d.kq);
      Exp2Arg eq[VN];
      double tq[VN];
#pragma unroll
      for (int k = 0; k < VN; ++k) {
        eq[k] = exp2_reduce(expo(xq[k], c256, xmcq));
        tq[k] = s_exp[eq[k].k & (kExpTable - 1)];
      }
#pragma unroll
      for (int k = 0; k < VN; ++k) sq += exp2_finish(eq[k], tq[k]);
    }
  } else {
    const double theta = d.theta * 256.0;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      float xq[VN], xp[VN];
      widen_raw<T>(vec(rq[i], i), xq);
      widen_raw<T>(vec(rp[i], i), xp);
      if (kMask) {
        mask_row<T>(xq, d.kq);
        mask_row<T>(xp, d.kp);
      }
      constexpr int HB = VN / 2;                  // entries per batch
#pragma unroll
      for (int h = 0; h < VN; h += HB) {
      Exp2Arg eq[HB], ep[HB];
      double tq[HB], tp[HB];
      bool act[HB];
#pragma unroll
      for (int k = 0; k < HB; ++k) {
        const double aq = expo(xq[h + k], c256, xmcq);
        const double ap = expo(xp[h + k], c256, xmcp);
        eq[k] = exp2_reduce(aq);
        ep[k] = exp2_reduce(ap);
        tq[k] = s_exp[eq[k].k & (kExpTable - 1)];
        tp[k] = s_exp[ep[k].k & (kExpTable - 1)];
        act[k] = aq - ap > theta;
      }
#pragma unroll
      for (int k = 0; k < HB; ++k) {
        const double wq = exp2_finish(eq[k], tq[k]);
        const double wp = exp2_finish(ep[k], tp[k]);
        sq += wq;
        sp += wp;
        // The normalisers in theta only decide which entries count as
        // q > coef p; an entry they misclassify has |q - coef p| ~ 1e-6 q, so
        // the masses move by ~1e-12.  (-inf - -inf is NaN: not counted,
        // weights are 0.)
        const double f = act[k] ? 1.0 : 0.0;
        sa = fma(wq, f, sa);
        sb = fma(wp, f, sb);
      }
      }
    }
  }
  sq = group8_sum_d(sq);
  sp = group8_sum_d(sp);
  sa = group8_sum_d(sa);
  sb = group8_sum_d(sb);
  if (s == 0) {
    const SubSums ss{sa, sb, sq, sp};
    SubSums* dst = csub + ((size_t)b * ncr + cr) * kSubPerChunk + sub_i;
    if (kAgent) {
      double* dd = reinterpret_cast<double*>(dst);
      st_agent_d(dd, sa); st_agent_d(dd + 1, sb); st_agent_d(dd + 2, sq); st_agent_d(dd + 3, sp);
    } else {
      *dst = ss;
    }
    s_sub[sub_i] = ss;
  }
  __syncthreads();
  // Chunk sums: one component per thread, sub-chunks in order.  Component
  // tid of ChunkSums {eq, ep, a, b} is component (tid + 2) % 4 of SubSums
  // {a, b, q, p}.
  if (tid < 4) {
    const int comp = (tid + 2) & 3;
    double acc = 0.0;
    for (int j = 0; j < kSubPerChunk; ++j) acc += reinterpret_cast<const double*>(&s_sub[j])[comp];
    double* dst = reinterpret_cast<double*>(csum + (size_t)b * ncr + cr) + tid;
    if (kAgent) st_agent_d(dst, acc);
    else *dst = acc;
  }
}

// The chain: every block first takes its sequence's decision itself (the
// same values in each; block 0 also stores it and emits greedy sequences),
// which saves a kernel boundary and a dependent read of the decision before
// the rows can be requested.  kDraw (ncr <= 64): the workgroup that completes
// a sequence's pass (its count in pcnt reaches ncr) then makes the final
// draw and emits, from the sums handed over as described above; otherwise
// k_locate does, in a kernel of its own.
template <typename T, bool kAligned, bool kMask = false, bool kDraw = false>
__global__ __launch_bounds__(kThreads, 4) void k_decide_residual(
    const T* __restrict__ tgt, const T* __restrict__ drf, const int32_t* __restrict__ dtok,
    const float* __restrict__ uni, const float* __restrict__ temp, int K, int V, int nc, int ncr,
    int force_greedy, const float2* __restrict__ part, const float* __restrict__ xd,
    const RowFilter* __restrict__ filt, int key16, Decision* __restrict__ dec,
    int32_t* __restrict__ out, int32_t* __restrict__ nacc, int32_t* __restrict__ kv_len,
    unsigned long long* counters, ChunkSums* __restrict__ csum, SubSums* __restrict__ csub,
    unsigned* __restrict__ pcnt) {
  const int b = blockIdx.x;
  const float t = temp_of(temp, b, force_greedy);
  if (!(t > 0.f) && blockIdx.y != 0) return;    // greedy: block 0 decides and emits; no pass
  const Decision d = decide_chain<kThreads>(b, dtok, uni, t, K, V, nc, part, xd, filt, key16,
                                            blockIdx.y == 0, dec, out, nacc, kv_len, counters);
  if (d.mode == kModeNone) return;
  __shared__ double s_exp[kExpTable];
  residual_pass<T, kAligned, kMask, kDraw>(tgt, drf, d, t, V, ncr, b, blockIdx.y, csum, csub, s_exp);
  if (!kDraw) return;
  __shared__ int s_last;
  vm_drain();
  __syncthreads();
  if (threadIdx.x == 0) s_last = atomicAdd(pcnt + b, 1u) + 1u == (unsigned)ncr ? 1 : 0;
  __syncthreads();
  if (!s_last) return;
  // Thread i < K emits draft i: it keeps its own token.
  const int my_draw = (int)threadIdx.x < K ? dtok[(size_t)b * K + threadIdx.x] : 0;
  const float u = uni[(size_t)b * (K + 1) + K];
  const int tok = locate_draw<T, true>(tgt, drf, d, u, t, V, ncr, csum + (size_t)b * ncr,
                                       csub + (size_t)b * ncr * kSubPerChunk, s_exp, false);
  emit_own(b, K, d.n, tok, my_draw, out, nacc, kv_len, counters);
}

// ---------------------------------------------------------------------------
// Tree verification.
// ---------------------------------------------------------------------------
// Outputs of a finished tree walk (threads 0..n-1 of the block): the final
// token after the path already written, -1 padding, the accepted count and
// the committed length.
__device__ __forceinline__ void emit_tree(int b, int N, int n, int tok, int32_t* __restrict__ out_tok,
                                          int32_t* __restrict__ out_node, int32_t* __restrict__ nacc,
                                          int32_t* __restrict__ kv_len, unsigned long long* counters) {
  const int i = threadIdx.x;
  if (i < N) {
    if (i >= n) out_tok[(size_t)b * N + i] = (i == n) ? tok : -1;
    if (i >= n) out_node[(size_t)b * N + i] = -1;
  }
  if (i == 0) {
    nacc[b] = n;
    kv_len[b] = kv_len[b] + n + 1;
    if (counters) {
      atomicAdd(&counters[0], (unsigned long long)(N - 1));
      atomicAdd(&counters[1], (unsigned long long)n);
    }
  }
}

// Walks sampling sequence b down from node v (n nodes accepted so far) with
// the sweep's statistics: the first child of every node is tested against q_v
// itself.  Accepted nodes are written to the outputs; the walk stops at the
// first rejection (a pass with coef = 1 follows) or at a leaf (the bonus
// pass from q_v follows).  One thread; rs(r) gives the merged statistics
// (raw max, sum) of swept row r; xd, tok and uni are this sequence's recorded
// logits [N][2], tokens [N] and uniforms [N], staged in LDS.
template <class RS>
__device__ void tree_walk(int b, int v, int n, const TreeShape& s, RS rs, const uint32_t* km,
                          const float* xd, const int* tok, const float* uni, float c, double cd,
                          int32_t* __restrict__ out_tok, int32_t* __restrict__ out_node,
                          Decision& dd, TreeState& st) {
  const int N = s.n;
  for (;;) {
    const int k0 = s.kid_off[v], k1 = s.kid_off[v + 1];
    const float2 rq = rs(v);
    if (k0 == k1) {
      dd = Decision{kModeQ, n, b * N + v, 0, rq.x, 0.f, 0.0, 0.0, 0.0, km[v], 0u};
      st = TreeState{v, 0, n, 1, 1.0};
      return;
    }
    const float2 rp = rs(N + s.int_idx[v]);
    const int ch = s.kids[k0];
    const float xq = xd[ch * 2], xp = xd[ch * 2 + 1];
    bool acc;
    if (xp == -INFINITY) {
      acc = true;                                   // p(d) == 0
    } else {
      // q/p in the log domain, as in the chain's accept tests.
      const double mq = (double)(rq.x * c), mp = (double)(rp.x * c);
      const double ly = ((double)xq * (double)c - mq) - ((double)xp * (double)c - mp);
      const double r = exp2(ly) * ((double)rp.y / (double)rq.y);
      acc = (double)uni[ch] < fmin(1.0, r);
    }
    if (acc) {
      out_node[(size_t)b * N + n] = ch;
      out_tok[(size_t)b * N + n] = tok[ch];
      ++n;
      v = ch;
      continue;
    }
    // Sweep normalisers moved to the exact pass's frame, for its q > p split.
    const double sq = (double)rq.y * exp2((double)(rq.x * c) - (double)rq.x * cd);
    const double sp = (double)rp.y * exp2((double)(rp.x * c) - (double)rp.x * cd);
    dd = Decision{kModeResid, n, b * N + v, b * N + v, rq.x, rp.x, log2(sq) - log2(sp), 1.0, 0.0,
                  km[v], km[N + s.int_idx[v]]};
    st = TreeState{v, 1, n, (k1 - k0 == 1) ? 1 : 0, 1.0};
    return;
  }
}

// ---------------------------------------------------------------------------
// k_tree_decide: grid (B); block 1024.  Merges the row statistics (kept in
// rowstat for the later rounds), finishes greedy sequences and starts the
// walk of sampling ones.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kDecideThreads) void k_tree_decide(
    const int32_t* __restrict__ tok, const float* __restrict__ uni, const float* __restrict__ temp,
    TreeShape s, const TreeShape* __restrict__ shapes, int RS, int V, int nc, int force_greedy,
    const float2* __restrict__ part,
    const RowFilter* __restrict__ filt, int key16, float* __restrict__ xd,
    float2* __restrict__ rowstat, Decision* __restrict__ dec, TreeState* __restrict__ state,
    int32_t* __restrict__ out_tok, int32_t* __restrict__ out_node, int32_t* __restrict__ nacc,
    int32_t* __restrict__ kv_len, unsigned long long* counters) {
  __shared__ float2 s_rs[2 * kMaxTree];
  __shared__ float s_xd[2 * kMaxTree], s_u[kMaxTree];
  __shared__ uint32_t s_km[2 * kMaxTree];
  __shared__ int s_tk[kMaxTree];
  __shared__ int s_n, s_tok;
  // The shape's tables in LDS: the walk looks them up with per-thread indices.
  // shapes: one per sequence (then s gives N only); RS: the rows per
  // sequence in part / rowstat / filt (a per-sequence shape may use fewer:
  // the statistics of the others are merged but never read).
  __shared__ TreeShape s_sh;
  const int b = blockIdx.x;
  if (threadIdx.x == 0) s_sh = shapes ? shapes[b] : s;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int N = s.n, R = RS;
  const float t = temp_of(temp, b, force_greedy);
  const bool greedy = !(t > 0.f);
  const int rows = greedy ? N : R;
  const float c = greedy ? 0.f : kLog2e / t;
  const float2* pb = part + (size_t)b * R * nc;
  // Every load at once: this sequence's tokens, uniforms and recorded logits
  // for the walk, and the row statistics (merged by 16-lane groups, 64 rows
  // per round).
  if (tid < N) s_tk[tid] = tok[(size_t)b * N + tid];
  if (!greedy && tid < N) s_u[tid] = uni[(size_t)b * N + tid];
  if (!greedy && tid < 2 * N) s_xd[tid] = xd[(size_t)b * N * 2 + tid];
  for (int r0 = 0; r0 < rows; r0 += kDecideThreads / 16) {
    const int r = r0 + (tid >> 4);
    const bool head = (tid & 15) == 0 && r < rows;
    // A filtered row: its law is renormalised over the kept set.
    const RowFilter rf = (filt && !greedy && head) ? filt[(size_t)b * R + r] : RowFilter{0u, 0u, 0.0};
    float a, bb;
    merge_row16(pb + (size_t)min(r, rows - 1) * nc, nc, greedy, c, tid & 15, a, bb);
    if (head) {
      s_rs[r] = make_float2(a, rf.key_min ? (float)rf.mass : bb);
      s_km[r] = rf.key_min;
    }
  }
  __syncthreads();
  if (filt && !greedy) {
    // A drafted token outside its parent's kept set has probability 0 there:
    // its recorded logit becomes -inf (the tests then read q(d) = 0 or
    // p(d) = 0), here and, written back, in the later rounds.
    if (tid < N) {
      const int v = tid;
      for (int k = s_sh.kid_off[v]; k < s_sh.kid_off[v + 1]; ++k) {
        const int ch = s_sh.kids[k];
        if (float_key(s_xd[ch * 2], key16 != 0) < s_km[v]) s_xd[ch * 2] = -INFINITY;
        if (float_key(s_xd[ch * 2 + 1], key16 != 0) < s_km[N + s_sh.int_idx[v]])
          s_xd[ch * 2 + 1] = -INFINITY;
      }
    }
    __syncthreads();
    if (tid < 2 * N) xd[(size_t)b * N * 2 + tid] = s_xd[tid];
  }
  if (!greedy && tid < R) rowstat[(size_t)b * R + tid] = s_rs[tid];
  if (tid == 0) {
    if (greedy) {
      // Follow the child whose token is the argmax of q_v (lowest index on
      // ties), the first such child in index order.
      int v = 0, n = 0, fin;
      for (;;) {
        const int am = __float_as_int(s_rs[v].y);
        int nxt = -1;
        for (int k = s_sh.kid_off[v]; k < s_sh.kid_off[v + 1]; ++k)
          if (clampi(s_tk[s_sh.kids[k]], 0, V - 1) == am) { nxt = s_sh.kids[k]; break; }
        if (nxt < 0) { fin = am; break; }
        out_node[(size_t)b * N + n] = nxt;
        out_tok[(size_t)b * N + n] = s_tk[nxt];
        ++n;
        v = nxt;
      }
      s_n = n;
      s_tok = fin;
      dec[b] = Decision{kModeNone, n, 0, 0, 0.f, 0.f, 0.0, 0.0, 0.0};
    } else {
      Decision dd;
      TreeState st;
      tree_walk(b, 0, 0, s_sh, [&](int r) { return s_rs[r]; }, s_km, s_xd, s_tk, s_u, c,
                kLog2eD / (double)t, out_tok, out_node, dd, st);
      dec[b] = dd;
      state[b] = st;
    }
  }
  if (greedy) {
    __syncthreads();
    emit_tree(b, N, s_n, s_tok, out_tok, out_node, nacc, kv_len, counters);
  }
}

// ---------------------------------------------------------------------------
// The step after a tree pass, for sequence b (a block of 256 threads, the one
// that completed the pass): the next sibling's test against the exact
// residual, which schedules the next pass (a further rejection, or a
// rejection or leaf below an accepted child), or the end of the walk, whose
// draw from this pass is left to k_tree_draw (the pass's sums stay in place:
// no later pass of the sequence overwrites them).  So a round waits for no
// draw, and all draws take one launch after the last round.  kAgent: the
// pass's chunk sums were stored by other workgroups of the running kernel.
// s: the shape in LDS (the walk indexes its tables per thread).
// ---------------------------------------------------------------------------
template <bool kAgent>
__device__ __forceinline__ void tree_step(
    int b, const int32_t* __restrict__ tok, const float* __restrict__ uni, const float* __restrict__ temp,
    const TreeShape& s, int RS, int ncr, int force_greedy, int last, const float2* __restrict__ rowstat,
    const RowFilter* __restrict__ filt, const float* __restrict__ xd,
    const ChunkSums* __restrict__ csum, Decision* __restrict__ dec, TreeState* __restrict__ state,
    int32_t* __restrict__ out_tok, int32_t* __restrict__ out_node, int32_t* __restrict__ nacc) {
  __shared__ float2 s_rs[2 * kMaxTree];
  __shared__ float s_xd[2 * kMaxTree], s_u[kMaxTree];
  __shared__ uint32_t s_km[2 * kMaxTree];
  __shared__ int s_tk[kMaxTree];
  __shared__ int s_draw, s_n;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = s.n, R = RS;
  // The walk's inputs, loaded together with the decision (one round trip).
  if (tid < R) {
    s_rs[tid] = rowstat[(size_t)b * R + tid];
    s_km[tid] = filt ? filt[(size_t)b * R + tid].key_min : 0u;
  }
  if (tid < N) {
    s_tk[tid] = tok[(size_t)b * N + tid];
    s_u[tid] = uni[(size_t)b * N + tid];
  }
  if (tid < 2 * N) s_xd[tid] = xd[(size_t)b * N * 2 + tid];
  const Decision d = dec[b];
  if (d.mode == kModeNone || d.mode == kModePending) return;
  const TreeState st = state[b];
  __syncthreads();
  const float t = temp_of(temp, b, force_greedy);
  const double cd = kLog2eD / (double)t;
  const ChunkSums* cg = csum + (size_t)b * ncr;
  if (wave == 0) {
    int draw = 1, n = st.n;
    if (!st.fin) {
      // The pass ran at coef after a rejection; its exact normalisers and the
      // residual mass Z (summed exactly as the draw sums it).
      const double sq = wave_chunk_sum(ncr, [&](int i) { return ld_sum(&cg[i].eq, kAgent); }, lane);
      const double sp = wave_chunk_sum(ncr, [&](int i) { return ld_sum(&cg[i].ep, kAgent); }, lane);
      const double isq = 1.0 / sq, isp = d.coef / sp;
      const double z = wave_chunk_sum(
          ncr, [&](int i) { return chunk_mass(ld_chunk_sums(cg + i, kAgent), kDrawResid, isq, isp); }, lane);
      if (lane == 0) {
        // A zero-mass residual leaves the law as it was.
        const bool frozen = !(z > 0.0);
        const double coef = frozen ? d.coef_prev : d.coef;
        const double zz = frozen ? st.n_prev : z;
        const int v = st.v, k0 = s.kid_off[v], nk = s.kid_off[v + 1] - k0;
        int pos = st.pos;
        for (;;) {
          const int ch = s.kids[k0 + pos];
          const float xq = s_xd[ch * 2], xp = s_xd[ch * 2 + 1];
          bool acc;
          if (xp == -INFINITY) {
            acc = true;
          } else {
            // q'(d) / p(d) = (q(d) / p(d) - coef)_+ / Z with the exact normalisers.
            const double lr = ((double)xq - (double)d.xmq) * cd - ((double)xp - (double)d.xmp) * cd;
            const double ratio = exp2(lr) * (sp / sq);
            const double r = fmax(0.0, ratio - coef) / zz;
            acc = (double)s_u[ch] < fmin(1.0, r);
          }
          if (acc) {
            out_node[(size_t)b * N + n] = ch;
            out_tok[(size_t)b * N + n] = s_tk[ch];
            Decision dd;
            TreeState ns;
            tree_walk(b, ch, n + 1, s, [&](int r) { return s_rs[r]; }, s_km, s_xd, s_tk, s_u, kLog2e / t,
                      cd, out_tok, out_node, dd, ns);
            dec[b] = dd;
            state[b] = ns;
            draw = 0;
            break;
          }
          ++pos;
          if (frozen) {
            if (pos < nk) continue;
            break;                                   // every child rejected: draw now
          }
          // Next residual step: coef grows by this pass's mass.
          Decision dd = d;
          dd.coef = d.coef + z;
          dd.coef_prev = d.coef;
          dd.theta = log2(dd.coef) + (log2(sq) - log2(sp));
          dec[b] = dd;
          state[b] = TreeState{v, pos, n, pos == nk ? 1 : 0, z};
          draw = 0;
          break;
        }
        if (!draw && last) {
          // The shape bounds the rounds, so this is unreachable; flag the
          // sequence rather than leave stale outputs.
          nacc[b] = -1;
          dec[b].mode = kModeNone;
        }
      }
      draw = __shfl(draw, 0, 64);
    }
    if (lane == 0) { s_draw = draw; s_n = n; }
  }
  __syncthreads();
  if (s_draw && tid == 0) {
    Decision pd = d;
    pd.draw_mode = d.mode;
    pd.mode = kModePending;
    pd.n = s_n;
    dec[b] = pd;
  }
}

// ---------------------------------------------------------------------------
// k_tree_round: grid (B, ncr); block 256.  One round of the tree walks: the
// pass each decision asks for (none for greedy, finished or pending
// sequences), then, in the workgroup that completes a sequence's pass (its
// count in rcnt reaches ncr), the step that follows.  That workgroup resets
// the count for the next round; k_sweep clears it before the first.
// ---------------------------------------------------------------------------
template <typename T, bool kAligned, bool kMask>
__global__ __launch_bounds__(kThreads, 4) void k_tree_round(
    const T* __restrict__ tgt, const T* __restrict__ drf, const int32_t* __restrict__ tok,
    const float* __restrict__ uni, const float* __restrict__ temp, TreeShape s,
    const TreeShape* __restrict__ shapes, int RS, int V, int ncr, int force_greedy, int last,
    const float2* __restrict__ rowstat,
    const RowFilter* __restrict__ filt, const float* __restrict__ xd,
    ChunkSums* __restrict__ csum, SubSums* __restrict__ csub, Decision* __restrict__ dec,
    TreeState* __restrict__ state, unsigned* __restrict__ rcnt, int32_t* __restrict__ out_tok,
    int32_t* __restrict__ out_node, int32_t* __restrict__ nacc) {
  __shared__ double s_exp[kExpTable];
  __shared__ int s_last;
  const int b = blockIdx.x;
  const Decision d = dec[b];
  if (d.mode == kModeNone || d.mode == kModePending) return;     // block-uniform
  residual_pass<T, kAligned, kMask, true>(tgt, drf, d, temp_of(temp, b, force_greedy), V, ncr, b,
                                          blockIdx.y, csum, csub, s_exp);
  vm_drain();
  __syncthreads();
  if (threadIdx.x == 0) s_last = atomicAdd(rcnt + b, 1u) + 1u == (unsigned)ncr ? 1 : 0;
  __syncthreads();
  if (!s_last) return;
  if (threadIdx.x == 0) __hip_atomic_store(rcnt + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // The shape's tables in LDS for the step (its walk indexes them per
  // thread; from the kernel arguments each lookup would be a memory load).
  __shared__ TreeShape s_sh;
  if (threadIdx.x == 0) s_sh = shapes ? shapes[b] : s;
  __syncthreads();
  tree_step<true>(b, tok, uni, temp, s_sh, RS, ncr, force_greedy, last, rowstat, filt, xd, csum, dec,
                  state, out_tok, out_node, nacc);
}

// k_tree_draw: grid (B); block 256.  The draws of the walks that ended in
// any round, each from the last pass of its sequence, then the outputs.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_tree_draw(
    const T* __restrict__ tgt, const T* __restrict__ drf, const float* __restrict__ uni,
    const float* __restrict__ temp, int N, int V, int ncr, int force_greedy,
    const ChunkSums* __restrict__ csum, const SubSums* __restrict__ csub,
    Decision* __restrict__ dec, int32_t* __restrict__ out_tok, int32_t* __restrict__ out_node,
    int32_t* __restrict__ nacc, int32_t* __restrict__ kv_len, unsigned long long* counters) {
  __shared__ double s_exp[kExpTable];
  const int b = blockIdx.x;
  if (force_greedy) return;                     // greedy walks finish in k_tree_decide
  const float t = temp[b];
  const float u = uni[(size_t)b * N];           // node 0's slot: the final draw
  Decision d = dec[b];
  // locate_draw reads d only after staging the sums; a sequence with no
  // pending draw comes back as -1.
  if (d.mode == kModePending) d.mode = d.draw_mode;
  else d.mode = kModeNone;
  const int tk = locate_draw<T>(tgt, drf, d, u, t, V, ncr, csum + (size_t)b * ncr,
                                csub + (size_t)b * ncr * kSubPerChunk, s_exp, true);
  if (tk < 0) return;
  emit_tree(b, N, d.n, tk, out_tok, out_node, nacc, kv_len, counters);
  if (threadIdx.x == 0) dec[b].mode = kModeNone;
}

struct RejectPlan {
  size_t part_off, csum_off, csub_off, dec_off, xd_off, filt_off, cnt_off, total;
  size_t partd_off, whist_off, wflag_off, wwin_off, fall_off, nfall_off, total_filtered;   // filtered bf16 calls only
};

// The window arrays of a filtered call over `rows` swept rows, from offset
// `at` on; returns the end.
template <class P>
static inline size_t win_plan(P& p, size_t at, size_t rows, int V) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t nc = (size_t)sweep_chunks(V), nblk = (nc + 3) / 4;
  p.partd_off = at;
  p.whist_off = p.partd_off + up(rows * nc * sizeof(double));
  p.wflag_off = p.whist_off + up(rows * nblk * kWinSlot * sizeof(uint16_t));
  p.wwin_off = p.wflag_off + up(rows * nblk * sizeof(uint32_t));
  p.fall_off = p.wwin_off + up(rows * sizeof(uint32_t));
  p.nfall_off = p.fall_off + up(rows * sizeof(uint32_t));
  return p.nfall_off + 256;
}

template <class P>
static inline WinArgs win_args(const P& p, char* ws, const int32_t* top_k, const float* top_p, int V) {
  return WinArgs{top_k, top_p, reinterpret_cast<double*>(ws + p.partd_off),
                 reinterpret_cast<uint16_t*>(ws + p.whist_off),
                 reinterpret_cast<uint32_t*>(ws + p.wflag_off),
                 reinterpret_cast<uint32_t*>(ws + p.wwin_off), reinterpret_cast<uint32_t*>(ws + p.fall_off),
                 reinterpret_cast<uint32_t*>(ws + p.nfall_off), (sweep_chunks(V) + 3) / 4};
}

static inline RejectPlan reject_plan(int B, int K, int V) {
  RejectPlan p{};
  const size_t R = 2 * (size_t)K + 1;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  p.part_off = 0;
  p.csum_off = up((size_t)B * R * sweep_chunks(V) * sizeof(float2));
  p.csub_off = p.csum_off + up((size_t)B * res_chunks(V) * sizeof(ChunkSums));
  p.dec_off = p.csub_off + up((size_t)B * res_chunks(V) * kSubPerChunk * sizeof(SubSums));
  p.xd_off = p.dec_off + up((size_t)B * sizeof(Decision));
  p.filt_off = p.xd_off + up((size_t)B * K * 2 * sizeof(float));
  p.cnt_off = p.filt_off + up((size_t)B * R * sizeof(RowFilter));
  p.total = p.cnt_off + up((size_t)B * sizeof(unsigned));
  p.total_filtered = win_plan(p, p.total, (size_t)B * R, V);
  return p;
}

template <typename T, bool kAligned>
static hipError_t launch_all(const void* tgt, const void* drf, const int32_t* dtok, const float* uni,
                             const float* temp, int32_t* out, int32_t* nacc, int32_t* kv_len,
                             unsigned long long* counters, int B, int K, int V, int force_greedy,
                             char* ws, hipStream_t st, const int32_t* top_k = nullptr,
                             const float* top_p = nullptr, bool win_ws = false) {
  const int nc = sweep_chunks(V);
  const int ncr = res_chunks(V);
  const int R = 2 * K + 1;
  const RejectPlan p = reject_plan(B, K, V);
  float2* part = reinterpret_cast<float2*>(ws + p.part_off);
  ChunkSums* csum = reinterpret_cast<ChunkSums*>(ws + p.csum_off);
  SubSums* csub = reinterpret_cast<SubSums*>(ws + p.csub_off);
  Decision* dec = reinterpret_cast<Decision*>(ws + p.dec_off);
  float* xd = reinterpret_cast<float*>(ws + p.xd_off);
  const T* t = static_cast<const T*>(tgt);
  const T* d = static_cast<const T*>(drf);
  unsigned* pcnt = reinterpret_cast<unsigned*>(ws + p.cnt_off);
  // Without draft logits every sequence is greedy: the grid holds the target
  // rows only (they come first in the sweep's order), and the decision one
  // workgroup per sequence.
  const bool filtered = (top_k || top_p) && !force_greedy;
  // Filtered bf16 rows (16-byte aligned) count their window in the sweep,
  // when the workspace holds the window arrays.
  const bool win = filtered && win_ws && kAligned && sizeof(T) == 2;
  const WinArgs wa = win ? win_args(p, ws, top_k, top_p, V) : WinArgs{};
  const dim3 sgrid(B * (force_greedy ? K + 1 : R), (nc + 3) / 4);
  if (win)
    hipLaunchKernelGGL((k_sweep<T, kAligned, ChainRows, true>), sgrid, dim3(kThreads), 0, st, t, d, dtok,
                       temp, ChainRows{K}, B, V, nc, force_greedy, part, xd, pcnt, wa);
  else
    hipLaunchKernelGGL((k_sweep<T, kAligned, ChainRows>), sgrid, dim3(kThreads), 0, st, t, d, dtok, temp,
                       ChainRows{K}, B, V, nc, force_greedy, part, xd, pcnt, WinArgs{});
  RowFilter* filt = filtered ? reinterpret_cast<RowFilter*>(ws + p.filt_off) : nullptr;
  // After the window, k_filter only takes the rows left on its list: two
  // blocks per CU (its occupancy) are one wave of launches.
  const int fgrid = win ? std::min(B * R, 2 * device_cus()) : B * R;
  if (win)
    hipLaunchKernelGGL((k_filter_win<ChainRows>), dim3(B * R), dim3(64), 0, st, temp, top_k,
                       top_p, ChainRows{K}, V, nc, force_greedy, part, filt, wa);
  if (filtered)
    if (win)
      hipLaunchKernelGGL((k_filter_list<T, kAligned, ChainRows>), dim3(fgrid), dim3(kFilterThreads), 0, st,
                         t, d, temp, top_k, top_p, ChainRows{K}, V, nc, force_greedy, part, filt, wa);
    else
      hipLaunchKernelGGL((k_filter<T, kAligned, ChainRows>), dim3(fgrid), dim3(kFilterThreads), 0, st, t,
                         d, temp, top_k, top_p, ChainRows{K}, V, nc, force_greedy, part, filt);
  const int key16 = sizeof(T) == 2 ? 1 : 0;
  // The draw joins the pass kernel while the chunk sums fit one wave.
  const bool fused = ncr <= 64;
  const dim3 grid(B, force_greedy ? 1 : ncr), block(kThreads);
  if (filtered && fused)
    hipLaunchKernelGGL((k_decide_residual<T, kAligned, true, true>), grid, block, 0, st, t, d, dtok, uni,
                       temp, K, V, nc, ncr, force_greedy, part, xd, filt, key16, dec, out, nacc, kv_len,
                       counters, csum, csub, pcnt);
  else if (filtered)
    hipLaunchKernelGGL((k_decide_residual<T, kAligned, true, false>), grid, block, 0, st, t, d, dtok,
                       uni, temp, K, V, nc, ncr, force_greedy, part, xd, filt, key16, dec, out, nacc,
                       kv_len, counters, csum, csub, pcnt);
  else if (fused)
    hipLaunchKernelGGL((k_decide_residual<T, kAligned, false, true>), grid, block, 0, st, t, d, dtok,
                       uni, temp, K, V, nc, ncr, force_greedy, part, xd, filt, key16, dec, out, nacc,
                       kv_len, counters, csum, csub, pcnt);
  else
    hipLaunchKernelGGL((k_decide_residual<T, kAligned, false, false>), grid, block, 0, st, t, d, dtok,
                       uni, temp, K, V, nc, ncr, force_greedy, part, xd, filt, key16, dec, out, nacc,
                       kv_len, counters, csum, csub, pcnt);
  if (!fused && !force_greedy)
    hipLaunchKernelGGL((k_locate<T>), dim3(B), dim3(kThreads), 0, st, t, d, dtok, uni, temp, K, V, ncr,
                       force_greedy, csum, csub, dec, out, nacc, kv_len, counters);
  return hipGetLastError();
}

// Tree workspace: the chain's arrays for up to 2N - 1 swept rows, plus the
// merged row statistics and the walk states.
struct TreePlan {
  size_t part_off, rowstat_off, csum_off, csub_off, dec_off, state_off, xd_off, rcnt_off, filt_off,
      shape_off, total;
  size_t partd_off, whist_off, wflag_off, wwin_off, fall_off, nfall_off, total_filtered;   // filtered bf16 calls only
};

static inline TreePlan tree_plan(int B, int N, int V) {
  TreePlan p{};
  const size_t R = 2 * (size_t)N - 1;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  p.part_off = 0;
  p.rowstat_off = up((size_t)B * R * sweep_chunks(V) * sizeof(float2));
  p.csum_off = p.rowstat_off + up((size_t)B * R * sizeof(float2));
  p.csub_off = p.csum_off + up((size_t)B * res_chunks(V) * sizeof(ChunkSums));
  p.dec_off = p.csub_off + up((size_t)B * res_chunks(V) * kSubPerChunk * sizeof(SubSums));
  p.state_off = p.dec_off + up((size_t)B * sizeof(Decision));
  p.xd_off = p.state_off + up((size_t)B * sizeof(TreeState));
  p.rcnt_off = p.xd_off + up((size_t)B * N * 2 * sizeof(float));
  p.filt_off = p.rcnt_off + up((size_t)B * sizeof(unsigned));
  p.shape_off = p.filt_off + up((size_t)B * R * sizeof(RowFilter));
  p.total = p.shape_off + up((size_t)B * sizeof(TreeShape));   // shapes: one per sequence
  p.total_filtered = win_plan(p, p.total, (size_t)B * R, V);
  return p;
}

// grid (ceil(B / 64)), block 64: sequence b's shape from its parent list
// parents[b] (one thread per sequence, tables built in LDS as on the host);
// a parent outside [0, i) is read as i - 1.
__global__ __launch_bounds__(64) void k_tree_shapes(const int32_t* __restrict__ parents, int B, int N,
                                                   TreeShape* __restrict__ shapes) {
  __shared__ TreeShape s_sh[64];
  __shared__ int8_t s_par[64][kMaxTree], s_fill[64][kMaxTree + 1];
  const int t = threadIdx.x, b = blockIdx.x * 64 + t;
  if (b >= B) return;
  TreeShape& s = s_sh[t];
  int8_t* par = s_par[t];
  int8_t* fill = s_fill[t];
  s = TreeShape{};
  s.n = N;
  for (int v = 0; v <= N; ++v) fill[v] = 0;
  par[0] = -1;
  for (int i = 1; i < N; ++i) {
    int pi = parents[(size_t)b * N + i];
    if (pi < 0 || pi >= i) pi = i - 1;
    par[i] = (int8_t)pi;
    ++fill[pi];
  }
  s.kid_off[0] = 0;
  for (int v = 0; v < N; ++v) s.kid_off[v + 1] = (int8_t)(s.kid_off[v] + fill[v]);
  for (int v = 0; v < N; ++v) fill[v] = s.kid_off[v];
  for (int i = 1; i < N; ++i) s.kids[fill[par[i]]++] = (int8_t)i;   // increasing index order
  s.n_int = 0;
  for (int v = 0; v < N; ++v) {
    s.int_idx[v] = -1;
    if (s.kid_off[v + 1] > s.kid_off[v]) {
      s.int_idx[v] = (int8_t)s.n_int;
      s.int_node[s.n_int++] = (int8_t)v;
    }
  }
  shapes[b] = s;
}

// Children lists of parent[] (parent[0] = -1, 0 <= parent[i] < i).
static inline bool build_shape(const int32_t* parent, int N, TreeShape& s) {
  if (N < 1 || N > kMaxTree || parent[0] != -1) return false;
  int cnt[kMaxTree] = {0};
  for (int i = 1; i < N; ++i) {
    if (parent[i] < 0 || parent[i] >= i) return false;
    ++cnt[parent[i]];
  }
  s = TreeShape{};
  s.n = N;
  s.kid_off[0] = 0;
  for (int v = 0; v < N; ++v) s.kid_off[v + 1] = (int8_t)(s.kid_off[v] + cnt[v]);
  int fill[kMaxTree];
  for (int v = 0; v < N; ++v) fill[v] = s.kid_off[v];
  for (int i = 1; i < N; ++i) s.kids[fill[parent[i]]++] = (int8_t)i;
  s.n_int = 0;
  for (int v = 0; v < N; ++v) {
    s.int_idx[v] = -1;
    if (cnt[v] > 0) {
      s.int_idx[v] = (int8_t)s.n_int;
      s.int_node[s.n_int++] = (int8_t)v;
    }
  }
  return true;
}

// The most exact passes a walk from v can need: each rejection among v's
// children costs one (the last one also serves the final draw), a leaf one
// (the bonus draw); accepting child j after j rejections continues there.
static int tree_rounds(const TreeShape& s, int v) {
  const int k0 = s.kid_off[v], m = s.kid_off[v + 1] - k0;
  if (m == 0) return 1;
  int best = m;
  for (int j = 0; j < m; ++j) best = std::max(best, j + tree_rounds(s, s.kids[k0 + j]));
  return best;
}

// shape: the batch's tree; or, with dparents ([B, N] device array), one tree
// per sequence (shape.n = N only), built on the device, the rows laid out
// for 2N - 1 per sequence, and N - 1 rounds (the most any tree of N nodes
// needs: a root with N - 1 children; a sequence whose walk has ended skips
// the rest).
template <typename T, bool kAligned>
static hipError_t launch_tree(const void* tgt, const void* drf, const TreeShape& shape,
                              const int32_t* dparents, const int32_t* tok, const float* uni,
                              const float* temp, int32_t* out_tok, int32_t* out_node, int32_t* nacc,
                              int32_t* kv_len, unsigned long long* counters, int B, int V,
                              int force_greedy, char* ws, hipStream_t st, const int32_t* top_k,
                              const float* top_p, bool win_ws) {
  const int N = shape.n;
  const int nc = sweep_chunks(V);
  const int ncr = res_chunks(V);
  const bool per_seq = dparents != nullptr;
  const int R = per_seq ? 2 * N - 1 : shape.n + shape.n_int;
  const TreePlan p = tree_plan(B, N, V);
  float2* part = reinterpret_cast<float2*>(ws + p.part_off);
  float2* rowstat = reinterpret_cast<float2*>(ws + p.rowstat_off);
  ChunkSums* csum = reinterpret_cast<ChunkSums*>(ws + p.csum_off);
  SubSums* csub = reinterpret_cast<SubSums*>(ws + p.csub_off);
  Decision* dec = reinterpret_cast<Decision*>(ws + p.dec_off);
  TreeState* state = reinterpret_cast<TreeState*>(ws + p.state_off);
  float* xd = reinterpret_cast<float*>(ws + p.xd_off);
  unsigned* rcnt = reinterpret_cast<unsigned*>(ws + p.rcnt_off);
  TreeShape* shapes = per_seq ? reinterpret_cast<TreeShape*>(ws + p.shape_off) : nullptr;
  const T* t = static_cast<const T*>(tgt);
  const T* d = static_cast<const T*>(drf);
  // Filters: thresholds and kept masses per swept row, as for the chain
  // (bf16 rows counted in a window by the sweep).
  const bool filtered = (top_k || top_p) && !force_greedy;
  const bool win = filtered && win_ws && kAligned && sizeof(T) == 2;
  const WinArgs wa = win ? win_args(p, ws, top_k, top_p, V) : WinArgs{};
  // Greedy only (no draft logits): the target rows, which come first.
  const dim3 sgrid(B * (force_greedy ? N : R), (nc + 3) / 4);
  if (per_seq) {
    hipLaunchKernelGGL(k_tree_shapes, dim3((B + 63) / 64), dim3(64), 0, st, dparents, B, N, shapes);
    if (win)
      hipLaunchKernelGGL((k_sweep<T, kAligned, TreeRowsSeq, true>), sgrid, dim3(kThreads), 0, st, t, d, tok,
                         temp, TreeRowsSeq{shapes, N}, B, V, nc, force_greedy, part, xd, rcnt, wa);
    else
      hipLaunchKernelGGL((k_sweep<T, kAligned, TreeRowsSeq>), sgrid, dim3(kThreads), 0, st, t, d, tok, temp,
                         TreeRowsSeq{shapes, N}, B, V, nc, force_greedy, part, xd, rcnt, WinArgs{});
  } else {
    if (win)
      hipLaunchKernelGGL((k_sweep<T, kAligned, TreeRows, true>), sgrid, dim3(kThreads), 0, st, t, d, tok,
                         temp, TreeRows{shape}, B, V, nc, force_greedy, part, xd, rcnt, wa);
    else
      hipLaunchKernelGGL((k_sweep<T, kAligned, TreeRows>), sgrid, dim3(kThreads), 0, st, t, d, tok, temp,
                         TreeRows{shape}, B, V, nc, force_greedy, part, xd, rcnt, WinArgs{});
  }
  RowFilter* filt = filtered ? reinterpret_cast<RowFilter*>(ws + p.filt_off) : nullptr;
  const int fgrid = win ? std::min(B * R, 2 * device_cus()) : B * R;
  if (win && per_seq)
    hipLaunchKernelGGL((k_filter_win<TreeRowsSeq>), dim3(B * R), dim3(64), 0, st, temp, top_k,
                       top_p, TreeRowsSeq{shapes, N}, V, nc, force_greedy, part, filt, wa);
  else if (win)
    hipLaunchKernelGGL((k_filter_win<TreeRows>), dim3(B * R), dim3(64), 0, st, temp, top_k,
                       top_p, TreeRows{shape}, V, nc, force_greedy, part, filt, wa);
  if (win && per_seq)
    hipLaunchKernelGGL((k_filter_list<T, kAligned, TreeRowsSeq>), dim3(fgrid), dim3(kFilterThreads), 0,
                       st, t, d, temp, top_k, top_p, TreeRowsSeq{shapes, N}, V, nc, force_greedy, part,
                       filt, wa);
  else if (win)
    hipLaunchKernelGGL((k_filter_list<T, kAligned, TreeRows>), dim3(fgrid), dim3(kFilterThreads), 0, st,
                       t, d, temp, top_k, top_p, TreeRows{shape}, V, nc, force_greedy, part, filt, wa);
  else if (filtered && per_seq)
    hipLaunchKernelGGL((k_filter<T, kAligned, TreeRowsSeq>), dim3(fgrid), dim3(kFilterThreads), 0, st,
                       t, d, temp, top_k, top_p, TreeRowsSeq{shapes, N}, V, nc, force_greedy, part, filt);
  else if (filtered)
    hipLaunchKernelGGL((k_filter<T, kAligned, TreeRows>), dim3(fgrid), dim3(kFilterThreads), 0, st, t,
                       d, temp, top_k, top_p, TreeRows{shape}, V, nc, force_greedy, part, filt);
  const int key16 = sizeof(T) == 2 ? 1 : 0;
  hipLaunchKernelGGL(k_tree_decide, dim3(B), dim3(kDecideThreads), 0, st, tok, uni, temp, shape, shapes,
                     R, V, nc, force_greedy, part, filt, key16, xd, rowstat, dec, state, out_tok,
                     out_node, nacc, kv_len, counters);
  const int rounds = force_greedy ? 0 : per_seq ? std::max(1, N - 1) : tree_rounds(shape, 0);
  for (int r = 1; r <= rounds; ++r) {
    if (filtered)
      hipLaunchKernelGGL((k_tree_round<T, kAligned, true>), dim3(B, ncr), dim3(kThreads), 0, st, t, d,
                         tok, uni, temp, shape, shapes, R, V, ncr, force_greedy, r == rounds ? 1 : 0,
                         rowstat, filt, xd, csum, csub, dec, state, rcnt, out_tok, out_node, nacc);
    else
      hipLaunchKernelGGL((k_tree_round<T, kAligned, false>), dim3(B, ncr), dim3(kThreads), 0, st, t, d,
                         tok, uni, temp, shape, shapes, R, V, ncr, force_greedy, r == rounds ? 1 : 0,
                         rowstat, filt, xd, csum, csub, dec, state, rcnt, out_tok, out_node, nacc);
  }
  if (rounds > 0)
    hipLaunchKernelGGL((k_tree_draw<T>), dim3(B), dim3(kThreads), 0, st, t, d, uni, temp, shape.n, V,
                       ncr, force_greedy, csum, csub, dec, out_tok, out_node, nacc, kv_len, counters);
  return hipGetLastError();
}

}  // namespace sv

extern "C" size_t spec_reject_sample_workspace_bytes(int B, int K, int V) {
  if (B <= 0 || K < 1 || K > SV_MAX_K || V < 1) return 0;
  return sv::reject_plan(B, K, V).total;
}

extern "C" size_t spec_reject_sample_filtered_workspace_bytes(int B, int K, int V) {
  if (B <= 0 || K < 1 || K > SV_MAX_K || V < 1) return 0;
  return sv::reject_plan(B, K, V).total_filtered;
}

static int reject_impl(const char* fn, const void* target_logits, const void* draft_logits,
                       const int32_t* draft_tokens, const float* uniforms, const float* temperature,
                       const int32_t* top_k, const float* top_p, int32_t* out_tokens,
                       int32_t* num_accepted, int32_t* kv_len, unsigned long long* counters, int B,
                       int K, int V, int dtype, void* workspace, size_t workspace_bytes,
                       void* hip_stream, bool allow_validate = true) {
  if (B < 0 || K < 1 || V < 1) return SV_ERR_INVALID_ARG;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_INVALID_ARG;
  if (K > SV_MAX_K) return SV_ERR_UNSUPPORTED;
  if ((long long)V >= (1LL << 31) / 4) return SV_ERR_UNSUPPORTED;
  // Grid limits: rows on x (31 bits), chunk groups and residual chunks on y (16 bits).
  if ((long long)B * (2 * K + 1) > 0x7fffffffLL || (sv::sweep_chunks(V) + 3) / 4 > 65535 ||
      sv::res_chunks(V) > 65535)
    return SV_ERR_UNSUPPORTED;
  if (B == 0) return SV_OK;
  if (!target_logits || !draft_tokens || !uniforms || !temperature || !out_tokens ||
      !num_accepted || !kv_len || !workspace)
    return SV_ERR_INVALID_ARG;
  // A filtered call given spec_reject_sample_filtered_workspace_bytes also
  // has room for the sweep's window; with the plain size it takes k_filter's
  // radix passes for every row.
  const sv::RejectPlan plan = sv::reject_plan(B, K, V);
  if (workspace_bytes < plan.total) return SV_ERR_WORKSPACE;
  const bool win_ws = workspace_bytes >= plan.total_filtered;
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return SV_ERR_INVALID_ARG;
  const int force_greedy = draft_logits == nullptr ? 1 : 0;
  const void* drf = draft_logits ? draft_logits : target_logits;   // never read when greedy
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  char* ws = static_cast<char*>(workspace);
  const uintptr_t align_bits = reinterpret_cast<uintptr_t>(target_logits) |
                               reinterpret_cast<uintptr_t>(drf);
  const bool chk = allow_validate && sv::validate_on();
  if (chk) {
    int s = sv::check_tokens(fn, draft_tokens, (long long)B * K, V, K, 0, st);
    if (s == SV_OK) s = sv::check_floats(fn, "uniforms", uniforms, (long long)B * (K + 1), true, st);
    if (s == SV_OK) s = sv::check_floats(fn, "temperature", temperature, B, false, st);
    if (s == SV_OK && top_p) s = sv::check_floats(fn, "top_p", top_p, B, false, st);
    if (s == SV_OK)
      s = sv::check_logits(fn, "target_logits", target_logits, (long long)B * (K + 1), V, dtype, st);
    if (s == SV_OK && draft_logits)
      s = sv::check_logits(fn, "draft_logits", draft_logits, (long long)B * K, V, dtype, st);
    if (s != SV_OK) return s;
  }
  hipError_t e;
  if (dtype == SV_BF16) {
    const bool al = (V % 8 == 0) && (align_bits & 15) == 0;
    e = al ? sv::launch_all<uint16_t, true>(target_logits, drf, draft_tokens, uniforms, temperature,
                                            out_tokens, num_accepted, kv_len, counters, B, K, V,
                                            force_greedy, ws, st, top_k, top_p, win_ws)
           : sv::launch_all<uint16_t, false>(target_logits, drf, draft_tokens, uniforms, temperature,
                                             out_tokens, num_accepted, kv_len, counters, B, K, V,
                                             force_greedy, ws, st, top_k, top_p, win_ws);
  } else {
    const bool al = (V % 4 == 0) && (align_bits & 15) == 0;
    e = al ? sv::launch_all<float, true>(target_logits, drf, draft_tokens, uniforms, temperature,
                                         out_tokens, num_accepted, kv_len, counters, B, K, V,
                                         force_greedy, ws, st, top_k, top_p, win_ws)
           : sv::launch_all<float, false>(target_logits, drf, draft_tokens, uniforms, temperature,
                                          out_tokens, num_accepted, kv_len, counters, B, K, V,
                                          force_greedy, ws, st, top_k, top_p, win_ws);
  }
  const int status = e == hipSuccess ? SV_OK : SV_ERR_HIP;
  return chk ? sv::finish(fn, st, status) : status;
}

extern "C" int spec_reject_sample(const void* target_logits, const void* draft_logits,
                                  const int32_t* draft_tokens, const float* uniforms,
                                  const float* temperature, int32_t* out_tokens,
                                  int32_t* num_accepted, int32_t* kv_len,
                                  unsigned long long* counters, int B, int K, int V, int dtype,
                                  void* workspace, size_t workspace_bytes, void* hip_stream) {
  return reject_impl("spec_reject_sample", target_logits, draft_logits, draft_tokens, uniforms,
                     temperature, nullptr,
                     nullptr, out_tokens, num_accepted, kv_len, counters, B, K, V, dtype, workspace,
                     workspace_bytes, hip_stream);
}

extern "C" int spec_reject_sample_filtered(const void* target_logits, const void* draft_logits,
                                           const int32_t* draft_tokens, const float* uniforms,
                                           const float* temperature, const int32_t* top_k,
                                           const float* top_p, int32_t* out_tokens,
                                           int32_t* num_accepted, int32_t* kv_len,
                                           unsigned long long* counters, int B, int K, int V,
                                           int dtype, void* workspace, size_t workspace_bytes,
                                           void* hip_stream) {
  return reject_impl("spec_reject_sample_filtered", target_logits, draft_logits, draft_tokens,
                     uniforms, temperature, top_k, top_p,
                     out_tokens, num_accepted, kv_len, counters, B, K, V, dtype, workspace,
                     workspace_bytes, hip_stream);
}

// ---------------------------------------------------------------------------
// spec_reject_sample_noalloc: spec_reject_sample with its workspace in a
// file-scope device array instead of a caller buffer, for callers that cannot
// allocate.  Each device holds its own copy of `scratch` (the runtime places
// it with the code object) until the process ends.  In host code `scratch`
// names a host-side stand-in, not the device copy: its device address is
// taken once per device with hipGetSymbolAddress, with that device current,
// and only that address is ever handed to a kernel.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};   // device address of `scratch`, per device

// The current device's copy of `scratch` (looked up on the first call made
// with that device current), or nullptr with *status set.
void* device_scratch(int* status) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *status = SV_ERR_HIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();   // the failure is reported here, not by a later call
      *status = SV_ERR_HIP;
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" int spec_reject_sample_noalloc(const void* target_logits, const void* draft_logits,
                                          const int32_t* draft_tokens, const float* uniforms,
                                          const float* temperature, int32_t* out_tokens,
                                          int32_t* num_accepted, int32_t* kv_len,
                                          unsigned long long* counters, int B, int K, int V,
                                          int dtype, void* hip_stream) {
  // Shape errors first, with the same codes as spec_reject_sample.
  if (B < 0 || K < 1 || V < 1) return SV_ERR_INVALID_ARG;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_INVALID_ARG;
  if (K > SV_MAX_K) return SV_ERR_UNSUPPORTED;
  if ((long long)V >= (1LL << 31) / 4) return SV_ERR_UNSUPPORTED;
  if (B == 0) return SV_OK;
  const size_t need = spec_reject_sample_workspace_bytes(B, K, V);
  if (need > (size_t)SV_NOALLOC_SCRATCH_BYTES) return SV_ERR_WORKSPACE;
  int status = SV_OK;
  void* ws = device_scratch(&status);
  if (!ws) return status;
  // The workspace needs no initial contents, so the array is not cleared.
  return reject_impl("spec_reject_sample_noalloc", target_logits, draft_logits, draft_tokens,
                     uniforms, temperature, nullptr, nullptr, out_tokens, num_accepted, kv_len,
                     counters, B, K, V, dtype, ws, need, hip_stream, false);
}

extern "C" size_t spec_reject_sample_tree_workspace_bytes(int B, int N, int V) {
  if (B <= 0 || N < 1 || N > sv::kMaxTree || V < 1) return 0;
  return sv::tree_plan(B, N, V).total;
}

extern "C" size_t spec_reject_sample_tree_filtered_workspace_bytes(int B, int N, int V) {
  if (B <= 0 || N < 1 || N > sv::kMaxTree || V < 1) return 0;
  return sv::tree_plan(B, N, V).total_filtered;
}

// per_seq false: parent is the batch's tree (host array); true: dparents
// holds one per sequence ([B, N] device array, NULL only for B == 0).
static int tree_impl(const char* fn, const void* target_logits, const void* draft_logits,
                     bool per_seq, const int32_t* parent, const int32_t* dparents,
                     const int32_t* tokens, const float* uniforms, const float* temperature,
                     const int32_t* top_k, const float* top_p, int32_t* out_tokens, int32_t* out_nodes,
                     int32_t* num_accepted, int32_t* kv_len, unsigned long long* counters, int B, int N,
                     int V, int dtype, void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (B < 0 || N < 1 || V < 1) return SV_ERR_INVALID_ARG;
  if (per_seq ? (B > 0 && !dparents) : !parent) return SV_ERR_INVALID_ARG;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_INVALID_ARG;
  if (N > sv::kMaxTree) return SV_ERR_UNSUPPORTED;
  sv::TreeShape shape{};
  shape.n = N;
  if (!per_seq && !sv::build_shape(parent, N, shape)) return SV_ERR_INVALID_ARG;
  if ((long long)V >= (1LL << 31) / 4) return SV_ERR_UNSUPPORTED;
  if ((long long)B * (2 * N - 1) > 0x7fffffffLL || (sv::sweep_chunks(V) + 3) / 4 > 65535 ||
      sv::res_chunks(V) > 65535)
    return SV_ERR_UNSUPPORTED;
  if (B == 0) return SV_OK;
  if (!target_logits || !tokens || !uniforms || !temperature || !out_tokens || !out_nodes ||
      !num_accepted || !kv_len || !workspace)
    return SV_ERR_INVALID_ARG;
  // As for the chain: the filtered size adds the sweep's window.
  const sv::TreePlan plan = sv::tree_plan(B, N, V);
  if (workspace_bytes < plan.total) return SV_ERR_WORKSPACE;
  const bool win_ws = workspace_bytes >= plan.total_filtered;
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return SV_ERR_INVALID_ARG;
  const int force_greedy = draft_logits == nullptr ? 1 : 0;
  const void* drf = draft_logits ? draft_logits : target_logits;   // never read when greedy
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  char* ws = static_cast<char*>(workspace);
  const uintptr_t align_bits = reinterpret_cast<uintptr_t>(target_logits) |
                               reinterpret_cast<uintptr_t>(drf);
  const bool chk = sv::validate_on();
  if (chk) {
    int s = sv::check_tokens(fn, tokens, (long long)B * N, V, N, 1, st);
    if (s == SV_OK) s = sv::check_floats(fn, "uniforms", uniforms, (long long)B * N, true, st);
    if (s == SV_OK) s = sv::check_floats(fn, "temperature", temperature, B, false, st);
    if (s == SV_OK && top_p) s = sv::check_floats(fn, "top_p", top_p, B, false, st);
    if (s == SV_OK)
      s = sv::check_logits(fn, "target_logits", target_logits, (long long)B * N, V, dtype, st);
    if (s == SV_OK && draft_logits)
      s = sv::check_logits(fn, "draft_logits", draft_logits, (long long)B * N, V, dtype, st);
    if (s == SV_OK && dparents) s = sv::check_parents(fn, dparents, B, N, st);
    if (s != SV_OK) return s;
  }
  hipError_t e;
  if (dtype == SV_BF16) {
    const bool al = (V % 8 == 0) && (align_bits & 15) == 0;
    e = al ? sv::launch_tree<uint16_t, true>(target_logits, drf, shape, dparents, tokens, uniforms,
                                             temperature, out_tokens, out_nodes, num_accepted, kv_len,
                                             counters, B, V, force_greedy, ws, st, top_k, top_p, win_ws)
           : sv::launch_tree<uint16_t, false>(target_logits, drf, shape, dparents, tokens, uniforms,
                                              temperature, out_tokens, out_nodes, num_accepted, kv_len,
                                              counters, B, V, force_greedy, ws, st, top_k, top_p, win_ws);
  } else {
    const bool al = (V % 4 == 0) && (align_bits & 15) == 0;
    e = al ? sv::launch_tree<float, true>(target_logits, drf, shape, dparents, tokens, uniforms,
                                          temperature, out_tokens, out_nodes, num_accepted, kv_len,
                                          counters, B, V, force_greedy, ws, st, top_k, top_p, win_ws)
           : sv::launch_tree<float, false>(target_logits, drf, shape, dparents, tokens, uniforms,
                                           temperature, out_tokens, out_nodes, num_accepted, kv_len,
                                           counters, B, V, force_greedy, ws, st, top_k, top_p, win_ws);
  }
  const int status = e == hipSuccess ? SV_OK : SV_ERR_HIP;
  return chk ? sv::finish(fn, st, status) : status;
}

extern "C" int spec_reject_sample_tree(const void* target_logits, const void* draft_logits,
                                       const int32_t* parent, const int32_t* tokens,
                                       const float* uniforms, const float* temperature,
                                       int32_t* out_tokens, int32_t* out_nodes,
                                       int32_t* num_accepted, int32_t* kv_len,
                                       unsigned long long* counters, int B, int N, int V, int dtype,
                                       void* workspace, size_t workspace_bytes, void* hip_stream) {
  return tree_impl("spec_reject_sample_tree", target_logits, draft_logits, false, parent, nullptr,
                   tokens, uniforms,
                   temperature, nullptr, nullptr, out_tokens, out_nodes, num_accepted, kv_len,
                   counters, B, N, V, dtype, workspace, workspace_bytes, hip_stream);
}

extern "C" int spec_reject_sample_tree_filtered(
    const void* target_logits, const void* draft_logits, const int32_t* parent,
    const int32_t* tokens, const float* uniforms, const float* temperature, const int32_t* top_k,
    const float* top_p, int32_t* out_tokens, int32_t* out_nodes, int32_t* num_accepted,
    int32_t* kv_len, unsigned long long* counters, int B, int N, int V, int dtype, void* workspace,
    size_t workspace_bytes, void* hip_stream) {
  return tree_impl("spec_reject_sample_tree_filtered", target_logits, draft_logits, false, parent, nullptr,
                   tokens, uniforms, temperature, top_k, top_p, out_tokens, out_nodes, num_accepted,
                   kv_len, counters, B, N, V, dtype, workspace, workspace_bytes, hip_stream);
}

extern "C" int spec_reject_sample_trees(
    const void* target_logits, const void* draft_logits, const int32_t* parents,
    const int32_t* tokens, const float* uniforms, const float* temperature, const int32_t* top_k,
    const float* top_p, int32_t* out_tokens, int32_t* out_nodes, int32_t* num_accepted,
    int32_t* kv_len, unsigned long long* counters, int B, int N, int V, int dtype, void* workspace,
    size_t workspace_bytes, void* hip_stream) {
  return tree_impl("spec_reject_sample_trees", target_logits, draft_logits, true, nullptr, parents,
                   tokens, uniforms, temperature, top_k, top_p, out_tokens, out_nodes, num_accepted,
                   kv_len, counters, B, N, V, dtype, workspace, workspace_bytes, hip_stream);
}
