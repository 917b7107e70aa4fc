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
// bf16 path (k_attn_mfma): one workgroup = 4 waves per (sequence, KV head,
// key split).  All G = Hq/Hkv query heads of the KV head and all K+1
// positions form the rows of one or two 32-row tiles, so each K/V byte is
// read once for the whole group.  Each wave walks page pairs (32 keys) of its
// split with its own online softmax:
//   S^T (32 keys x 32 rows) = K . Q^T   8 x v_mfma_f32_32x32x16_bf16 (D=128)
//   O^T (32 d x 32 rows)   += V^T . P^T 2 x 4 MFMAs per pair
// The MFMA key order is permuted so that the C registers of S^T are exactly
// the B operand of the P.V product (lane l holds tokens 8*(l/32)..+7 of each
// page for row l%32), and so that every K and V load is a 16-byte vector with
// the 64 lanes of one instruction reading 512 contiguous bytes from each page.
// No LDS is touched in the key loop; the 4 waves merge through LDS at the end.
// Splits are merged by k_attn_combine (log-sum-exp weights, fixed order).
//
// fp32 path (k_attn_valu): plain VALU kernel, one wave per query row; used for
// fp32 caches (the correctness configuration).

#include "common.h"

namespace sv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kAttnThreads = 256;
constexpr int kPairKeys = 32;

// Keys per split for the bf16 path, chosen from the launch shape alone so the
// workspace size is a pure function of the arguments.
static inline int attn_split_keys(int B, int Hkv, int max_len) {
  const long long work = (long long)max_len * B * Hkv;
  long long per = work / 4096;                 // aim for ~4096 workgroup slots
  per = (per + 127) / 128 * 128;               // whole page pairs for all 4 waves
  if (per < 128) per = 128;
  if (per > (1 << 20)) per = 1 << 20;
  return (int)per;
}

static inline int attn_tiles(int G, int K1) { return (G * K1 + 31) / 32; }

// ---------------------------------------------------------------------------
// bf16 MFMA kernel.  grid (nsplit, Hkv, B), block 256.
// Partials: opart[((b*Hkv + g)*nsplit + s)*rows_pad*D + row*D + d] (fp32,
// scaled to the split max) and ml[(b*Hkv + g)*nsplit + s)*rows_pad + row] =
// (max, sum), base-2 scaled scores.
// ---------------------------------------------------------------------------
template <int D, int NT>
__global__ __launch_bounds__(kAttnThreads) void k_attn_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ kv_len, uint16_t* __restrict__ out,
    int K1, int Hq, int Hkv, int num_blocks, int mbps, int split_keys, int nsplit, float sl2,
    float* __restrict__ opart, float2* __restrict__ ml) {
  constexpr int KK = D / 16;         // MFMA k-steps for S
  constexpr int DT = D / 32;         // d tiles for O
  constexpr int ROWS = 32 * NT;
  constexpr int OPAD = D + 4;        // LDS row stride (floats)
  __shared__ float s_o[4][32][OPAD];
  __shared__ float s_m[4][ROWS], s_l[4][ROWS];

  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = Hq / Hkv;
  const int rows = G * K1;
  const int L0 = kv_len[b];
  const int L = L0 + K1;
  // kv_len above the max_kv_len the grid was sized for is a precondition
  // violation: its extra keys are dropped, never read out of bounds.
  const int my_splits = min(nsplit, (L + split_keys - 1) / split_keys);
  if (split >= my_splits) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;

  // Q operand (B of S^T = K Q^T): lane holds Q[row = nt*32 + l32][kk*16 + hh*8 .. +8].
  bf16x8 qf[NT][KK];
  int lim[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int row = nt * 32 + l32;
    const bool valid = row < rows;
    const int hq = valid ? row / K1 : 0;
    const int i = valid ? row - hq * K1 : K1 - 1;
    lim[nt] = L0 + i;                             // last visible key
    const uint16_t* qp = q + (((size_t)b * K1 + i) * Hq + (size_t)g * G + hq) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if (valid) {
        qf[nt][kk] = *reinterpret_cast<const bf16x8*>(qp + kk * 16 + hh * 8);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[nt][kk][e] = (__bf16)0.f;
      }
    }
  }

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

  // K operand row of this lane: MFMA key mk = l32 -> page mk>>4, token below.
  const int k_page = l32 >> 4;
  const int k_tok = 8 * ((l32 >> 2) & 1) + 4 * ((l32 >> 3) & 1) + (l32 & 3);
  const size_t page_elems = (size_t)D * 16;
  const int32_t* btb = bt + (size_t)b * mbps;

  const int npairs = (L + kPairKeys - 1) / kPairKeys;
  const int split_pairs = split_keys / kPairKeys;
  const int p_lo = split * split_pairs;
  const int p_hi = min(npairs, p_lo + split_pairs);

  for (int pr = p_lo + wave; pr < p_hi; pr += 4) {
    int blk[2];
#pragma unroll
    for (int sg = 0; sg < 2; ++sg) {
      const int pg = min(2 * pr + sg, mbps - 1);
      blk[sg] = clampi(btb[pg], 0, num_blocks - 1);
    }
    const uint16_t* kpage = kc + ((size_t)blk[k_page] * Hkv + g) * page_elems;
    bf16x8 kf[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      kf[kk] = *reinterpret_cast<const bf16x8*>(kpage + ((2 * kk + hh) * 16 + k_tok) * 8);
    bf16x8 vf[2][DT];
#pragma unroll
    for (int sg = 0; sg < 2; ++sg) {
      const uint16_t* vpage = vc + ((size_t)blk[sg] * Hkv + g) * page_elems;
#pragma unroll
      for (int j = 0; j < DT; ++j)
        vf[sg][j] = *reinterpret_cast<const bf16x8*>(vpage + (32 * j + l32) * 16 + 8 * hh);
    }
    const int key0 = pr * kPairKeys + 8 * hh;     // key of reg r: key0 + (r>>3)*16 + (r&7)
    if (pr * kPairKeys + kPairKeys > L) {
      // Slots past the sequence end may hold anything (even NaN); their
      // probability is 0, but 0 * NaN would still reach O, so zero them.
#pragma unroll
      for (int sg = 0; sg < 2; ++sg)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (key0 + sg * 16 + e >= L)
#pragma unroll
            for (int j = 0; j < DT; ++j) vf[sg][j][e] = (__bf16)0.f;
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x16 s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qf[nt][kk], s, 0, 0, 0);
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + (r >> 3) * 16 + (r & 7);
        const float v = (key <= lim[nt]) ? s[r] * sl2 : -INFINITY;
        s[r] = v;
        mx = fmaxf(mx, v);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run[nt], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2_dev(m_run[nt] - m_use);
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = exp2_dev(s[r] - m_use);
        rs += s[r];
      }
      rs += __shfl_xor(rs, 32, 64);
      l_run[nt] = l_run[nt] * alpha + rs;
      m_run[nt] = m_new;
      bf16x8 pf[2];
#pragma unroll
      for (int sg = 0; sg < 2; ++sg)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[sg][e] = (__bf16)s[8 * sg + e];
#pragma unroll
      for (int j = 0; j < DT; ++j) {
#pragma unroll
        for (int r = 0; r < 16; ++r) o[nt][j][r] *= alpha;
#pragma unroll
        for (int sg = 0; sg < 2; ++sg)
          o[nt][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[sg][j], pf[sg], o[nt][j], 0, 0, 0);
      }
    }
  }

  // Merge the 4 waves, one 32-row tile at a time, then write the output (one
  // split) or this split's partial.
  const int G_rows = rows;
  const size_t part_base = ((size_t)(b * Hkv + g) * nsplit + split) * ROWS;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (lane < 32) { s_m[wave][nt * 32 + l32] = m_run[nt]; s_l[wave][nt * 32 + l32] = l_run[nt]; }
    __syncthreads();
    float mall = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) mall = fmaxf(mall, s_m[w][nt * 32 + l32]);
    const float muse = (mall == -INFINITY) ? 0.f : mall;
    const float f = exp2_dev(m_run[nt] - muse);
#pragma unroll
    for (int j = 0; j < DT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = 32 * j + 8 * (r >> 2) + 4 * hh + (r & 3);
        s_o[wave][l32][d] = o[nt][j][r] * f;
      }
    __syncthreads();
    // 256 threads: row = tid / 8, 16 consecutive d per thread (D = 128) or 8 (D = 64).
    constexpr int DPT = D / 8;
    const int row_l = tid >> 3;
    const int d0 = (tid & 7) * DPT;
    const int row = nt * 32 + row_l;
    float mrow = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) mrow = fmaxf(mrow, s_m[w][row]);
    const float mu = (mrow == -INFINITY) ? 0.f : mrow;
    float lsum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) lsum += s_l[w][row] * exp2_dev(s_m[w][row] - mu);
    float acc[DPT];
#pragma unroll
    for (int e = 0; e < DPT; ++e) acc[e] = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int e = 0; e < DPT; ++e) acc[e] += s_o[w][row_l][d0 + e];
    if (row < G_rows) {
      if (my_splits == 1) {
        const int hq = row / K1, i = row - hq * K1;
        uint16_t* op = out + (((size_t)b * K1 + i) * Hq + (size_t)g * G + hq) * D + d0;
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
        for (int e = 0; e < DPT; e += 2) {
          const __bf16 lo = (__bf16)(acc[e] * inv);
          const __bf16 hi = (__bf16)(acc[e + 1] * inv);
          const uint32_t w = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                             ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
          *reinterpret_cast<uint32_t*>(op + e) = w;
        }
      } else {
        float* pp = opart + (part_base + row) * D + d0;
#pragma unroll
        for (int e = 0; e < DPT; e += 4)
          *reinterpret_cast<float4*>(pp + e) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
        if ((tid & 7) == 0) ml[part_base + row] = make_float2(mrow, lsum);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Split combine.  grid (Hkv, B), block 256: row = tid / 8, D/8 d's per thread.
// ---------------------------------------------------------------------------
template <int D, int NT>
__global__ __launch_bounds__(kAttnThreads) void k_attn_combine(
    const float* __restrict__ opart, const float2* __restrict__ ml, const int32_t* __restrict__ kv_len,
    uint16_t* __restrict__ out, int K1, int Hq, int Hkv, int split_keys, int nsplit) {
  constexpr int ROWS = 32 * NT;
  constexpr int DPT = D / 8;
  const int g = blockIdx.x, b = blockIdx.y;
  const int L = kv_len[b] + K1;
  const int my_splits = min(nsplit, (L + split_keys - 1) / split_keys);
  if (my_splits <= 1) return;
  const int G = Hq / Hkv;
  const int rows = G * K1;
  const int tid = threadIdx.x;
  const int d0 = (tid & 7) * DPT;
  for (int row = tid >> 3; row < ROWS; row += kAttnThreads / 8) {
    if (row >= rows) break;
    const size_t base = (size_t)(b * Hkv + g) * nsplit * ROWS + row;
    float m = -INFINITY;
    for (int s = 0; s < my_splits; ++s) m = fmaxf(m, ml[base + (size_t)s * ROWS].x);
    const float mu = (m == -INFINITY) ? 0.f : m;
    float lsum = 0.f;
    float acc[DPT];
#pragma unroll
    for (int e = 0; e < DPT; ++e) acc[e] = 0.f;
    for (int s = 0; s < my_splits; ++s) {
      const float2 st = ml[base + (size_t)s * ROWS];
      const float f = exp2_dev(st.x - mu);
      lsum += st.y * f;
      const float* pp = opart + (base + (size_t)s * ROWS) * D + d0;
#pragma unroll
      for (int e = 0; e < DPT; e += 4) {
        const float4 v = *reinterpret_cast<const float4*>(pp + e);
        acc[e] += v.x * f; acc[e + 1] += v.y * f; acc[e + 2] += v.z * f; acc[e + 3] += v.w * f;
      }
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const int hq = row / K1, i = row - hq * K1;
    uint16_t* op = out + (((size_t)b * K1 + i) * Hq + (size_t)g * G + hq) * D + d0;
#pragma unroll
    for (int e = 0; e < DPT; e += 2) {
      const __bf16 lo = (__bf16)(acc[e] * inv);
      const __bf16 hi = (__bf16)(acc[e + 1] * inv);
      const uint32_t w = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                         ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
      *reinterpret_cast<uint32_t*>(op + e) = w;
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 VALU kernel: grid (K1, Hq, B), block 64 (one wave per query row).
// k_cache [NB, Hkv, D/4, 16, 4], v_cache [NB, Hkv, D, 16].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_attn_valu(
    const float* __restrict__ q, const float* __restrict__ kc, const float* __restrict__ vc,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ kv_len, float* __restrict__ out,
    int K1, int Hq, int Hkv, int D, int num_blocks, int mbps, float sl2) {
  __shared__ float s_q[256];
  __shared__ float s_p[64];
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int g = h / (Hq / Hkv);
  const int t = kv_len[b] + i;                    // last visible key
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
    if (j <= t) {
      const int blk = clampi(btb[min(j >> 4, mbps - 1)], 0, num_blocks - 1);
      const float* kp = kc + ((size_t)blk * Hkv + g) * page;
      const int tok = j & 15;
      float acc = 0.f;
      for (int d = 0; d < D; ++d) acc += s_q[d] * kp[((d >> 2) * 16 + tok) * 4 + (d & 3)];
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
      const int blk = clampi(btb[min(jk >> 4, mbps - 1)], 0, num_blocks - 1);
      const float* vp = vc + ((size_t)blk * Hkv + g) * page;
      const float pj = s_p[jj];
      for (int c = 0; c < 4; ++c) {
        const int d = lane + 64 * c;
        if (d < D) o[c] += pj * vp[d * 16 + (jk & 15)];
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

struct AttnPlan {
  int split_keys, nsplit, tiles;
  size_t opart_bytes, ml_bytes;
};

static inline AttnPlan attn_plan(int B, int K, int Hq, int Hkv, int D, int max_kv_len) {
  AttnPlan p{};
  const int K1 = K + 1;
  const int max_len = max_kv_len + K1;
  p.split_keys = attn_split_keys(B, Hkv, max_len);
  p.nsplit = (max_len + p.split_keys - 1) / p.split_keys;
  p.tiles = attn_tiles(Hq / Hkv, K1);
  const size_t parts = (size_t)B * Hkv * p.nsplit * 32 * p.tiles;
  p.opart_bytes = p.nsplit > 1 ? ((parts * D * sizeof(float) + 255) & ~(size_t)255) : 0;
  p.ml_bytes = p.nsplit > 1 ? ((parts * sizeof(float2) + 255) & ~(size_t)255) : 0;
  return p;
}

template <int D, int NT>
static hipError_t launch_mfma(const void* q, const void* kc, const void* vc, const int32_t* bt,
                              const int32_t* kv_len, void* out, int B, int K1, int Hq, int Hkv,
                              int num_blocks, int mbps, float sl2, const AttnPlan& p, char* ws,
                              hipStream_t st) {
  float* opart = reinterpret_cast<float*>(ws);
  float2* ml = reinterpret_cast<float2*>(ws + p.opart_bytes);
  hipLaunchKernelGGL((k_attn_mfma<D, NT>), dim3(p.nsplit, Hkv, B), dim3(kAttnThreads), 0, st,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kc),
                     static_cast<const uint16_t*>(vc), bt, kv_len, static_cast<uint16_t*>(out), K1, Hq,
                     Hkv, num_blocks, mbps, p.split_keys, p.nsplit, sl2, opart, ml);
  if (p.nsplit > 1)
    hipLaunchKernelGGL((k_attn_combine<D, NT>), dim3(Hkv, B), dim3(kAttnThreads), 0, st, opart, ml,
                       kv_len, static_cast<uint16_t*>(out), K1, Hq, Hkv, p.split_keys, p.nsplit);
  return hipGetLastError();
}

}  // namespace sv

extern "C" size_t spec_verify_attn_workspace_bytes(int B, int K, int Hq, int Hkv, int D,
                                                   int max_kv_len) {
  if (B <= 0 || K < 1 || Hq < 1 || Hkv < 1 || D < 1 || max_kv_len < 0) return 0;
  const sv::AttnPlan p = sv::attn_plan(B, K, Hq, Hkv, D, max_kv_len);
  return p.opart_bytes + p.ml_bytes;
}

extern "C" int spec_verify_attn(const void* q, const void* k_cache, const void* v_cache,
                                const int32_t* block_table, const int32_t* kv_len, void* out, int B,
                                int K, int Hq, int Hkv, int D, int block_size, int num_blocks,
                                int max_blocks_per_seq, int max_kv_len, float scale, int dtype,
                                void* workspace, size_t workspace_bytes, void* hip_stream) {
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
  if (B > 65535 || Hkv > 65535) return SV_ERR_UNSUPPORTED;
  const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)D);
  const float sl2 = sc * sv::kLog2e;
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  const int K1 = K + 1;
  hipError_t e;
  if (dtype == SV_F32) {
    hipLaunchKernelGGL(sv::k_attn_valu, dim3(K1, Hq, B), dim3(64), 0, st,
                       static_cast<const float*>(q), static_cast<const float*>(k_cache),
                       static_cast<const float*>(v_cache), block_table, kv_len,
                       static_cast<float*>(out), K1, Hq, Hkv, D, num_blocks, max_blocks_per_seq, sl2);
    e = hipGetLastError();
  } else {
    const sv::AttnPlan p = sv::attn_plan(B, K, Hq, Hkv, D, max_kv_len);
    if (p.opart_bytes + p.ml_bytes > 0) {
      if (!workspace) return SV_ERR_INVALID_ARG;
      if (workspace_bytes < p.opart_bytes + p.ml_bytes) return SV_ERR_WORKSPACE;
      if (reinterpret_cast<uintptr_t>(workspace) & 255) return SV_ERR_INVALID_ARG;
    }
    const uintptr_t al = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) |
                         reinterpret_cast<uintptr_t>(v_cache) | reinterpret_cast<uintptr_t>(out);
    if (al & 15) return SV_ERR_INVALID_ARG;
    char* ws = static_cast<char*>(workspace);
    if (D == 128) {
      e = p.tiles == 1 ? sv::launch_mfma<128, 1>(q, k_cache, v_cache, block_table, kv_len, out, B, K1,
                                                 Hq, Hkv, num_blocks, max_blocks_per_seq, sl2, p, ws, st)
                       : sv::launch_mfma<128, 2>(q, k_cache, v_cache, block_table, kv_len, out, B, K1,
                                                 Hq, Hkv, num_blocks, max_blocks_per_seq, sl2, p, ws, st);
    } else {
      e = p.tiles == 1 ? sv::launch_mfma<64, 1>(q, k_cache, v_cache, block_table, kv_len, out, B, K1,
                                                Hq, Hkv, num_blocks, max_blocks_per_seq, sl2, p, ws, st)
                       : sv::launch_mfma<64, 2>(q, k_cache, v_cache, block_table, kv_len, out, B, K1,
                                                Hq, Hkv, num_blocks, max_blocks_per_seq, sl2, p, ws, st);
    }
  }
  return e == hipSuccess ? SV_OK : SV_ERR_HIP;
}
