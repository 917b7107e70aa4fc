// Lossless rejection-sampling verifier over the full vocabulary, plus the
// commit of the logical KV length.
//
// Method: AI Engineering from Scratch, "Speculative decoding and EAGLE-3" --
// "Concept" (accept d ~ p with probability min(1, q(d)/p(d)); on rejection
// draw from (q - p)_+ normalised; bonus token from q_{N+1} when every draft
// passes), "Build it" steps 1-2 (p(d) <= 0 accepts; a zero-mass residual falls
// back to q) and "Rolling back the KV cache" (logical length reset).
//
// Three kernels on the caller's stream:
//   k_sweep   one pass over every logit row (the HBM-bound part): per 4096-
//             entry chunk, the raw maximum and sum_v 2^(x_v c - m) in fp32
//             (c = log2(e) / T), or the chunk argmax for greedy sequences.
//             16-byte coalesced loads, one wave per chunk, butterfly
//             reductions, no LDS.  These statistics feed the accept tests,
//             whose decisions are only sensitive at the 1e-5 level.
//   k_decide  per (sequence, 8192-entry chunk): merge the row statistics in a
//             fixed order, run the accept tests and the first-rejection scan
//             (every block of a sequence redundantly and bit-identically),
//             then summarise its chunk of the one row pair the final draw
//             needs (target and draft row n, or target row K for the bonus)
//             in float64: sum e_q, sum e_p, and the same two sums over the
//             entries with q > p, with e = 2^((x - xmax) c) from the float64
//             exp2.  Those four sums give both the exact normalisers and the
//             residual mass of the chunk, so the row pair is read once here.
//             Greedy sequences are finished here.
//   k_locate  per sampling sequence: float64 prefix over the chunk masses,
//             pick the chunk holding u_K * Z, stage its float64 weights in LDS,
//             scan them, emit the tokens and commit kv_len.
// The final draw is therefore computed to ~1e-14 in probability mass, so it
// agrees with a float64 reference except within a vanishing band around the
// CDF edges.  No floating-point atomics and fixed merge orders: results are
// bitwise reproducible run to run.

// Contraction off: the weights recomputed by k_locate must equal the ones of
// k_decide bit for bit, and merges must stay symmetric in their operands.
// Fused multiply-adds that are wanted are written out.
#pragma clang fp contract(off)

#include "common.h"

namespace sv {

constexpr int kThreads = 256;
constexpr int kSweepChunk = 4096;   // elements per wave in k_sweep
constexpr int kResChunk = 8192;     // elements per block in k_decide / k_locate
constexpr int kMaxRows = 2 * SV_MAX_K + 1;
constexpr int kPartStage = 4096;    // row statistics staged in LDS per sequence (32 KB)
constexpr double kLog2eD = 1.4426950408889634074;

struct Decision {
  int n;          // accepted drafts
  float xmq;      // raw maximum of target row n
  float xmp;      // raw maximum of draft row n (unused when n == K)
  float pad;
};

struct ChunkSums {
  double eq, ep;  // sum of e_q, e_p over the chunk
  double a, b;    // the same sums over entries with q > p
};

// The same sums for each 256-entry sub-chunk (a, b as above, q = sum e_q);
// the final draw narrows chunk -> sub-chunk -> entry.
constexpr int kSub = 256;
constexpr int kSubPerChunk = kResChunk / kSub;
struct SubSums {
  double a, b, q;
};

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

// ---------------------------------------------------------------------------
// k_sweep: grid (B * (2K+1), ceil(nc / 4)); block 256 = 4 waves, one chunk each.
// part[row * nc + chunk] = (raw max, sum 2^(x c - fl(max c))) or, greedy,
// (max value, argmax index bits).
// ---------------------------------------------------------------------------
template <typename T, bool kAligned>
__global__ __launch_bounds__(kThreads) void k_sweep(
    const T* __restrict__ tgt, const T* __restrict__ drf, const float* __restrict__ temp,
    int K, int V, int nc, int force_greedy, float2* __restrict__ part) {
  const int R = 2 * K + 1;
  const int row = blockIdx.x;
  const int b = row / R;
  const int j = row - b * R;
  const float t = temp_of(temp, b, force_greedy);
  const bool greedy = !(t > 0.f);
  if (greedy && j > K) return;                 // greedy never reads draft rows
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int chunk = blockIdx.y * 4 + wave;
  if (chunk >= nc) return;
  const T* src = (j <= K) ? tgt + ((size_t)b * (K + 1) + j) * (size_t)V
                          : drf + ((size_t)b * K + (j - K - 1)) * (size_t)V;
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

// Merge the nc chunk statistics of one row (one wave, fixed order).
// Sampling rows give (raw max, sum relative to fl(raw max * c)).
__device__ __forceinline__ void merge_row(const float2* __restrict__ pr, int nc, bool greedy, float c,
                                          int lane, float& a, float& bb) {
  if (greedy) {
    float v = -INFINITY;
    int i = INT32_MAX;
    for (int k = lane; k < nc; k += 64) {
      const float2 p = pr[k];
      am_merge(v, i, p.x, __float_as_int(p.y));
    }
    wave_am_reduce(v, i);
    a = v;
    bb = __int_as_float(i);
  } else {
    float m = -INFINITY, s = 0.f, xr = -INFINITY;
    for (int k = lane; k < nc; k += 64) {
      const float2 p = pr[k];
      ms_merge(m, s, p.x * c, p.y);
      xr = fmaxf(xr, p.x);
    }
    wave_ms_reduce(m, s);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) xr = fmaxf(xr, __shfl_xor(xr, off, 64));
    a = xr;
    bb = s;
  }
}

__device__ __forceinline__ void emit(int b, int K, int n, int tok, const int32_t* __restrict__ dtok,
                                     int32_t* __restrict__ out, int32_t* __restrict__ nacc,
                                     int32_t* __restrict__ kv_len, unsigned long long* counters) {
  for (int i = 0; i <= K; ++i) {
    int v = -1;
    if (i < n) v = dtok[(size_t)b * K + i];
    else if (i == n) v = tok;
    out[(size_t)b * (K + 1) + i] = v;
  }
  nacc[b] = n;
  kv_len[b] = kv_len[b] + n + 1;
  if (counters) {
    atomicAdd(&counters[0], (unsigned long long)K);
    atomicAdd(&counters[1], (unsigned long long)n);
  }
}

// Float64 2^a for a <= 0, to a few ulp, at a fraction of the library
// routine's cost.  With k = round(-16 a) (taken with the 2^52 + 2^51 shifter,
// whose low word then holds k), 2^a = 2^(-k/16) * 2^r where r = a + k/16 is
// exact and |r| <= 1/32.  2^(-k/16) comes from a table the block fills with
// the device's float64 exp2; 2^r is the Taylor series of e^(r ln 2) to degree
// 7, Horner form in r (first dropped term < 2e-18).  Arguments below -64 are
// clamped there: such entries weigh < 5.4e-20 of the row maximum (whose
// weight is 1), far below every tolerance; -inf gives exactly 0.
constexpr int kExpTable = 1025;                  // 2^(-k/16), k = 0..1024

__device__ __forceinline__ void fill_exp_table(double* tab) {
  for (int k = threadIdx.x; k < kExpTable; k += blockDim.x) tab[k] = exp2(-(double)k * 0.0625);
}

__device__ __forceinline__ double exp2_neg(double a, const double* __restrict__ tab) {
  const double ac = fmax(a, -64.0);
  const double shifter = 6755399441055744.0;               // 2^52 + 2^51
  const double t = fma(ac, -16.0, shifter);                // shifter + k
  const int k = __double2loint(t);
  const double r = fma(t - shifter, 0.0625, ac);           // a + k/16, exact
  double p = 1.5252733804059838e-05;                       // ln2^7 / 7!
  p = fma(p, r, 1.5403530393381606e-04);                   // ln2^6 / 6!
  p = fma(p, r, 1.3333558146428441e-03);                   // ln2^5 / 5!
  p = fma(p, r, 9.618129107628477e-03);                   // ln2^4 / 4!
  p = fma(p, r, 5.5504108664821576e-02);                   // ln2^3 / 3!
  p = fma(p, r, 2.402265069591007e-01);                   // ln2^2 / 2!
  p = fma(p, r, 6.931471805599453e-01);                   // ln2
  p = fma(p, r, 1.0);
  const double v = tab[k] * p;
  return (a == -INFINITY) ? 0.0 : v;
}

// Unnormalised float64 weight 2^((x - xmax) c) of one entry (x <= xmax).
__device__ __forceinline__ double expw(float x, double xmax, double c, const double* __restrict__ tab) {
  return exp2_neg(((double)x - xmax) * c, tab);
}

__device__ __forceinline__ double wave_sum_d(double x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// ---------------------------------------------------------------------------
// k_decide: grid (B, ncr); block 256.
// ---------------------------------------------------------------------------
template <typename T, bool kAligned>
__global__ __launch_bounds__(kThreads) void k_decide(
    const T* __restrict__ tgt, const T* __restrict__ drf, const int32_t* __restrict__ dtok,
    const float* __restrict__ uni, const float* __restrict__ temp, int K, int V, int nc, int ncr,
    int force_greedy, const float2* __restrict__ part, ChunkSums* __restrict__ csum,
    SubSums* __restrict__ csub, Decision* __restrict__ dec, int32_t* __restrict__ out,
    int32_t* __restrict__ nacc, int32_t* __restrict__ kv_len, unsigned long long* counters) {
  __shared__ float s_a[kMaxRows], s_b[kMaxRows];
  __shared__ float2 s_part[kPartStage];
  __shared__ float s_xq[SV_MAX_K], s_xp[SV_MAX_K];
  __shared__ int s_d[SV_MAX_K];
  __shared__ int s_n;
  __shared__ double s_red[4][kThreads / 64];
  __shared__ double s_exp[kExpTable];
  const int b = blockIdx.x;
  const int cr = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int R = 2 * K + 1;
  const float t = temp_of(temp, b, force_greedy);
  const bool greedy = !(t > 0.f);
  const int rows = greedy ? K + 1 : R;
  const float c = greedy ? 0.f : kLog2e / t;
  // All independent loads first: the row statistics of this sequence (into
  // LDS when they fit) and the drafted tokens' logits.
  const float2* pb = part + (size_t)b * R * nc;
  const bool staged = rows * nc <= kPartStage;
  if (staged)
    for (int k = tid; k < rows * nc; k += kThreads) s_part[k] = pb[k];
  if (!greedy) fill_exp_table(s_exp);
  if (tid < K) {
    const int d = clampi(dtok[(size_t)b * K + tid], 0, V - 1);
    s_d[tid] = d;
    if (!greedy) {
      s_xq[tid] = Vec16<T>::one(tgt + ((size_t)b * (K + 1) + tid) * (size_t)V + d);
      s_xp[tid] = Vec16<T>::one(drf + ((size_t)b * K + tid) * (size_t)V + d);
    }
  }
  __syncthreads();
  for (int r = wave; r < rows; r += kThreads / 64) {
    float a, bb;
    merge_row(staged ? s_part + r * nc : pb + (size_t)r * nc, nc, greedy, c, lane, a, bb);
    if (lane == 0) { s_a[r] = a; s_b[r] = bb; }
  }
  __syncthreads();
  if (tid == 0) {
    int n = 0;
    for (int i = 0; i < K; ++i) {
      const int d = s_d[i];
      bool acc;
      if (greedy) {
        acc = (d == __float_as_int(s_b[i]));
      } else {
        const float xq = s_xq[i];
        const float xp = s_xp[i];
        if (xp == -INFINITY) {
          acc = true;                                   // p(d) == 0
        } else {
          // q/p = 2^((xq c - mq) - (xp c - mp)) * sp / sq with m = fl(xmax c),
          // taken in the log domain so small probabilities do not underflow.
          const double mq = (double)(s_a[i] * c), mp = (double)(s_a[K + 1 + i] * c);
          const double ly = ((double)xq * (double)c - mq) - ((double)xp * (double)c - mp);
          const double r = exp2(ly) * ((double)s_b[K + 1 + i] / (double)s_b[i]);
          acc = (double)uni[(size_t)b * (K + 1) + i] < fmin(1.0, r);
        }
      }
      if (!acc) break;
      ++n;
    }
    s_n = n;
    if (greedy) {
      if (cr == 0) emit(b, K, n, __float_as_int(s_b[n]), dtok, out, nacc, kv_len, counters);
    } else if (cr == 0) {
      Decision dd;
      dd.n = n;
      dd.xmq = s_a[n];
      dd.xmp = (n < K) ? s_a[K + 1 + n] : 0.f;
      dd.pad = 0.f;
      dec[b] = dd;
    }
  }
  __syncthreads();
  if (greedy) return;
  const int n = s_n;
  const bool bonus = (n == K);
  const double cd = kLog2eD / (double)t;
  const float xmq = s_a[n];
  const float xmp = bonus ? 0.f : s_a[K + 1 + n];
  // Approximate normalisers (sweep precision, moved to the 2^((x - xmax) c)
  // reference) only decide which entries count as q > p; an entry they
  // misclassify has |q - p| ~ 1e-6 q, so the chunk masses move by ~1e-12.
  const double sq_approx = (double)s_b[n] * exp2((double)(xmq * c) - (double)xmq * cd);
  const double sp_approx =
      bonus ? 1.0 : (double)s_b[K + 1 + n] * exp2((double)(xmp * c) - (double)xmp * cd);
  const T* trow = tgt + ((size_t)b * (K + 1) + n) * (size_t)V;
  const T* drow = bonus ? trow : drf + ((size_t)b * K + n) * (size_t)V;
  constexpr int VN = Vec16<T>::N;
  constexpr int IT = kResChunk / (kThreads * VN);
  constexpr int kSubLanes = kSub / VN;            // lanes covering one sub-chunk per step
  const int lo = cr * kResChunk;
  const double xmqd = (double)xmq, xmpd = (double)xmp;
  SubSums* sub = csub + ((size_t)b * ncr + cr) * kSubPerChunk;
  double eq = 0.0, ep = 0.0, sa = 0.0, sb = 0.0;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int e = lo + it * kThreads * VN + tid * VN;
    float xq[VN], xp[VN];
    load_vec<T, kAligned>(trow, e, V, xq);
    if (!bonus) load_vec<T, kAligned>(drow, e, V, xp);
    double tq = 0.0, ta = 0.0, tb = 0.0;
#pragma unroll
    for (int k = 0; k < VN; ++k) {
      if (e + k < V) {
        const double wq = expw(xq[k], xmqd, cd, s_exp);
        tq += wq;
        if (!bonus) {
          const double wp = expw(xp[k], xmpd, cd, s_exp);
          ep += wp;
          if (wq * sp_approx > wp * sq_approx) { ta += wq; tb += wp; }
        }
      }
    }
    eq += tq;
    sa += ta;
    sb += tb;
    // Sub-chunk sums: kSubLanes consecutive lanes cover one 256-entry run.
#pragma unroll
    for (int off = kSubLanes / 2; off > 0; off >>= 1) {
      tq += __shfl_xor(tq, off, 64);
      ta += __shfl_xor(ta, off, 64);
      tb += __shfl_xor(tb, off, 64);
    }
    if ((lane & (kSubLanes - 1)) == 0)
      sub[it * (kThreads * VN / kSub) + (tid * VN) / kSub] = SubSums{ta, tb, tq};
  }
  eq = wave_sum_d(eq);
  ep = wave_sum_d(ep);
  sa = wave_sum_d(sa);
  sb = wave_sum_d(sb);
  if (lane == 0) { s_red[0][wave] = eq; s_red[1][wave] = ep; s_red[2][wave] = sa; s_red[3][wave] = sb; }
  __syncthreads();
  if (tid == 0) {
    ChunkSums cs{0.0, 0.0, 0.0, 0.0};
    for (int w = 0; w < kThreads / 64; ++w) {
      cs.eq += s_red[0][w]; cs.ep += s_red[1][w]; cs.a += s_red[2][w]; cs.b += s_red[3][w];
    }
    csum[(size_t)b * ncr + cr] = cs;
  }
}

// ---------------------------------------------------------------------------
// k_locate: grid (B); block 256.  Sampling sequences only.  Narrows the draw
// chunk -> sub-chunk (from the stored sums) -> entry (exact weights of one
// 256-entry run, one per thread, scanned in fixed order).
// ---------------------------------------------------------------------------
__device__ __forceinline__ double chunk_mass(const ChunkSums& cs, bool qonly, double isq, double isp) {
  return qonly ? cs.eq * isq : fmax(0.0, cs.a * isq - cs.b * isp);
}
__device__ __forceinline__ double sub_mass(const SubSums& ss, bool qonly, double isq, double isp) {
  return qonly ? ss.q * isq : fmax(0.0, ss.a * isq - ss.b * isp);
}

template <typename T, bool kAligned>
__global__ __launch_bounds__(kThreads) void k_locate(
    const T* __restrict__ tgt, const T* __restrict__ drf, const int32_t* __restrict__ dtok,
    const float* __restrict__ uni, const float* __restrict__ temp, int K, int V, int ncr,
    int force_greedy, const ChunkSums* __restrict__ csum, const SubSums* __restrict__ csub,
    const Decision* __restrict__ dec, int32_t* __restrict__ out, int32_t* __restrict__ nacc,
    int32_t* __restrict__ kv_len, unsigned long long* counters) {
  static_assert(kSub == kThreads, "one sub-chunk entry per thread");
  __shared__ ChunkSums s_cs[kThreads];
  __shared__ SubSums s_ss[kSubPerChunk];
  __shared__ double s_exp[kExpTable];
  __shared__ double s_wtot[kThreads / 64];
  __shared__ int s_chunk, s_sub, s_fallback, s_useq, s_first, s_lastpos;
  __shared__ double s_base, s_target, s_isq, s_isp;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float t = temp_of(temp, b, force_greedy);
  if (!(t > 0.f)) return;
  const double cd = kLog2eD / (double)t;
  const Decision d = dec[b];
  const int n = d.n;
  const bool bonus = (n == K);
  // Chunk sums are loaded in parallel, then walked in order by thread 0.
  const ChunkSums* cg = csum + (size_t)b * ncr;
  const bool cstaged = ncr <= kThreads;
  if (cstaged && tid < ncr) s_cs[tid] = cg[tid];
  fill_exp_table(s_exp);
  __syncthreads();
  if (tid == 0) {
    const ChunkSums* cs = cstaged ? s_cs : cg;
    double sq = 0.0, sp = 0.0;
    for (int i = 0; i < ncr; ++i) { sq += cs[i].eq; sp += cs[i].ep; }
    const double isq = 1.0 / sq;
    const double isp = bonus ? 0.0 : 1.0 / sp;
    double z = 0.0;
    for (int i = 0; i < ncr; ++i) z += chunk_mass(cs[i], bonus, isq, isp);
    const bool useq = !bonus && !(z > 0.0);                  // zero-mass residual: draw from q
    const bool qonly = bonus || useq;
    if (useq) { z = 0.0; for (int i = 0; i < ncr; ++i) z += chunk_mass(cs[i], true, isq, isp); }
    const double target = (double)uni[(size_t)b * (K + 1) + K] * z;
    double p = 0.0, base = 0.0;
    int ch = -1;
    for (int i = 0; i < ncr; ++i) {
      const double p2 = p + chunk_mass(cs[i], qonly, isq, isp);
      if (p2 > target) { ch = i; base = p; break; }
      p = p2;
    }
    int fb = 0;
    if (ch < 0) {                                             // rounding at u -> 1
      fb = 1;
      for (int i = ncr - 1; i >= 0; --i)
        if (chunk_mass(cs[i], qonly, isq, isp) > 0.0) { ch = i; break; }
      if (ch < 0) ch = 0;
    }
    s_chunk = ch; s_fallback = fb; s_useq = useq ? 1 : 0;
    s_base = base; s_target = target; s_isq = isq; s_isp = isp;
    s_first = INT32_MAX; s_lastpos = -1;
  }
  __syncthreads();
  const int ch = s_chunk;
  const bool qonly = bonus || (s_useq != 0);
  const double isq = s_isq, isp = s_isp;
  if (tid < kSubPerChunk) s_ss[tid] = csub[((size_t)b * ncr + ch) * kSubPerChunk + tid];
  __syncthreads();
  if (tid == 0) {
    int sc = -1;
    double p = s_base, base = s_base;
    if (!s_fallback) {
      for (int j = 0; j < kSubPerChunk; ++j) {
        const double p2 = p + sub_mass(s_ss[j], qonly, isq, isp);
        if (p2 > s_target) { sc = j; base = p; break; }
        p = p2;
      }
    }
    if (sc < 0) {                                             // no crossing left: last positive run
      s_fallback = 1;
      for (int j = kSubPerChunk - 1; j >= 0; --j)
        if (sub_mass(s_ss[j], qonly, isq, isp) > 0.0) { sc = j; break; }
      if (sc < 0) sc = 0;
    }
    s_sub = sc;
    s_base = base;
  }
  __syncthreads();
  const T* trow = tgt + ((size_t)b * (K + 1) + n) * (size_t)V;
  const T* drow = bonus ? trow : drf + ((size_t)b * K + n) * (size_t)V;
  const int e = ch * kResChunk + s_sub * kSub + tid;
  double w = 0.0;
  if (e < V) {
    const double q = expw(Vec16<T>::one(trow + e), (double)d.xmq, cd, s_exp) * isq;
    w = qonly ? q : fmax(0.0, q - expw(Vec16<T>::one(drow + e), (double)d.xmp, cd, s_exp) * isp);
  }
  // Inclusive prefix over the 256 entries in vocabulary order: a wave scan
  // plus the totals of the waves before (fixed order).
  double incl = w;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) s_wtot[wave] = incl;
  __syncthreads();
  double run = s_base + incl;
  for (int ww = 0; ww < wave; ++ww) run += s_wtot[ww];
  if (!s_fallback && run > s_target) atomicMin(&s_first, e);
  if (w > 0.0) atomicMax(&s_lastpos, e);
  __syncthreads();
  if (tid == 0) {
    int tok = s_first;
    if (tok == INT32_MAX) tok = s_lastpos;                   // no crossing: last positive weight
    if (tok < 0) tok = clampi(ch * kResChunk + s_sub * kSub, 0, V - 1);
    emit(b, K, n, tok, dtok, out, nacc, kv_len, counters);
  }
}

struct RejectPlan {
  size_t part_off, csum_off, csub_off, dec_off, total;
};

static inline RejectPlan reject_plan(int B, int K, int V) {
  RejectPlan p{};
  const size_t R = 2 * (size_t)K + 1;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  p.part_off = 0;
  p.csum_off = up((size_t)B * R * sweep_chunks(V) * sizeof(float2));
  p.csub_off = p.csum_off + up((size_t)B * res_chunks(V) * sizeof(ChunkSums));
  p.dec_off = p.csub_off + up((size_t)B * res_chunks(V) * kSubPerChunk * sizeof(SubSums));
  p.total = p.dec_off + up((size_t)B * sizeof(Decision));
  return p;
}

template <typename T, bool kAligned>
static hipError_t launch_all(const void* tgt, const void* drf, const int32_t* dtok, const float* uni,
                             const float* temp, int32_t* out, int32_t* nacc, int32_t* kv_len,
                             unsigned long long* counters, int B, int K, int V, int force_greedy,
                             char* ws, hipStream_t st) {
  const int nc = sweep_chunks(V);
  const int ncr = res_chunks(V);
  const int R = 2 * K + 1;
  const RejectPlan p = reject_plan(B, K, V);
  float2* part = reinterpret_cast<float2*>(ws + p.part_off);
  ChunkSums* csum = reinterpret_cast<ChunkSums*>(ws + p.csum_off);
  SubSums* csub = reinterpret_cast<SubSums*>(ws + p.csub_off);
  Decision* dec = reinterpret_cast<Decision*>(ws + p.dec_off);
  const T* t = static_cast<const T*>(tgt);
  const T* d = static_cast<const T*>(drf);
  hipLaunchKernelGGL((k_sweep<T, kAligned>), dim3(B * R, (nc + 3) / 4), dim3(kThreads), 0, st, t, d,
                     temp, K, V, nc, force_greedy, part);
  hipLaunchKernelGGL((k_decide<T, kAligned>), dim3(B, ncr), dim3(kThreads), 0, st, t, d, dtok, uni,
                     temp, K, V, nc, ncr, force_greedy, part, csum, csub, dec, out, nacc, kv_len, counters);
  hipLaunchKernelGGL((k_locate<T, kAligned>), dim3(B), dim3(kThreads), 0, st, t, d, dtok, uni, temp,
                     K, V, ncr, force_greedy, csum, csub, dec, out, nacc, kv_len, counters);
  return hipGetLastError();
}

}  // namespace sv

extern "C" size_t spec_reject_sample_workspace_bytes(int B, int K, int V) {
  if (B <= 0 || K < 1 || K > SV_MAX_K || V < 1) return 0;
  return sv::reject_plan(B, K, V).total;
}

extern "C" int spec_reject_sample(const void* target_logits, const void* draft_logits,
                                  const int32_t* draft_tokens, const float* uniforms,
                                  const float* temperature, int32_t* out_tokens,
                                  int32_t* num_accepted, int32_t* kv_len,
                                  unsigned long long* counters, int B, int K, int V, int dtype,
                                  void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (B < 0 || K < 1 || V < 1) return SV_ERR_INVALID_ARG;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_INVALID_ARG;
  if (K > SV_MAX_K) return SV_ERR_UNSUPPORTED;
  if ((long long)V >= (1LL << 31) / 4) return SV_ERR_UNSUPPORTED;
  if ((long long)B * (2 * K + 1) > 0x7fffffffLL || (V + 16383) / 16384 > 65535)
    return SV_ERR_UNSUPPORTED;
  if (B == 0) return SV_OK;
  if (!target_logits || !draft_tokens || !uniforms || !temperature || !out_tokens ||
      !num_accepted || !kv_len || !workspace)
    return SV_ERR_INVALID_ARG;
  if (workspace_bytes < spec_reject_sample_workspace_bytes(B, K, V)) return SV_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return SV_ERR_INVALID_ARG;
  const int force_greedy = draft_logits == nullptr ? 1 : 0;
  const void* drf = draft_logits ? draft_logits : target_logits;   // never read when greedy
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  char* ws = static_cast<char*>(workspace);
  const uintptr_t align_bits = reinterpret_cast<uintptr_t>(target_logits) |
                               reinterpret_cast<uintptr_t>(drf);
  hipError_t e;
  if (dtype == SV_BF16) {
    const bool al = (V % 8 == 0) && (align_bits & 15) == 0;
    e = al ? sv::launch_all<uint16_t, true>(target_logits, drf, draft_tokens, uniforms, temperature,
                                            out_tokens, num_accepted, kv_len, counters, B, K, V,
                                            force_greedy, ws, st)
           : sv::launch_all<uint16_t, false>(target_logits, drf, draft_tokens, uniforms, temperature,
                                             out_tokens, num_accepted, kv_len, counters, B, K, V,
                                             force_greedy, ws, st);
  } else {
    const bool al = (V % 4 == 0) && (align_bits & 15) == 0;
    e = al ? sv::launch_all<float, true>(target_logits, drf, draft_tokens, uniforms, temperature,
                                         out_tokens, num_accepted, kv_len, counters, B, K, V,
                                         force_greedy, ws, st)
           : sv::launch_all<float, false>(target_logits, drf, draft_tokens, uniforms, temperature,
                                          out_tokens, num_accepted, kv_len, counters, B, K, V,
                                          force_greedy, ws, st);
  }
  return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}
