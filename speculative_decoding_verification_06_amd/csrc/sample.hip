// The acceptance rule over the vocabulary, after the target pass.
//
//   rowstats : combine per-unit (max, sum exp) of each logits row (one
//              unit per LM-head work group) into softmax(l / T), and the
//              per-unit sums of each draft row into
//              q' = q^(1/T) / sum ("Speculative decoding" pigeon guide, When it
//              breaks: the same temperature / top-p on p and q)
//   topp     : nucleus of each row by a radix select (11, 11, 10-bit
//              digits) on an order-preserving key, with masses in 2^-40
//              fixed point so the histogram sums are exact and order
//              independent
//   decide   : ratio test r * q'(x) < p'(x) per drafted position, first
//              rejection per sequence, then the chunk sums of the resample
//              row (lattice-ai-eng explainer, acceptance
//              rule; pigeon guide, How it works, step 3); at T = 0 the draft
//              is compared to the argmax
//   resample : inverse CDF over max(0, p' - q') at the first rejection, or
//              over p' for the bonus slot or a zero residual (pigeon guide,
//              steps 4-5; scalablesystem article, The Accept/Reject
//              Mechanism), as per-chunk sums plus one chunk rescan
//
// Floating-point contraction is off in this file so every kernel that
// evaluates p'(v) or the residual gets the same bits.

#include <climits>

#include "common.h"
#include "internal.h"

#pragma clang fp contract(off)

namespace sv {

enum { RI_M = 0, RI_INVZ = 1, RI_THR = 2, RI_TIE = 3, RI_INVZN = 4, RI_NUC = 5 };
constexpr int kRowInfo = 8;

__device__ __forceinline__ uint32_t q_key(float qv) { return qv > 0.f ? __float_as_uint(qv) : 0u; }

__device__ __forceinline__ bool in_nucleus(const float* ri, uint32_t key, int v) {
  const uint32_t thr = __float_as_uint(ri[RI_THR]);
  return key > thr || (key == thr && v <= __float_as_int(ri[RI_TIE]));
}

// p'(v) of a logits row (T > 0).
__device__ __forceinline__ float p_prime(const float* ri, float l, int v, float invT) {
  float p = expf((l - ri[RI_M]) * invT) * ri[RI_INVZ];
  if (__float_as_int(ri[RI_NUC])) p = in_nucleus(ri, logit_key(l), v) ? p * ri[RI_INVZN] : 0.f;
  return p;
}

// Pre-nucleus q'(v); tmode 1 (T == 1) divides by the row sum directly.
__device__ __forceinline__ float q_tempered(const float* ri, float qv, int tmode, float invT) {
  if (tmode == 1) return qv * ri[RI_INVZ];
  return qv > 0.f ? expf(logf(qv) * invT - ri[RI_M]) * ri[RI_INVZ] : 0.f;
}

__device__ __forceinline__ float q_prime(const float* ri, float qv, int v, int tmode, float invT) {
  float w = q_tempered(ri, qv, tmode, invT);
  if (__float_as_int(ri[RI_NUC])) w = in_nucleus(ri, q_key(qv), v) ? w * ri[RI_INVZN] : 0.f;
  return w;
}

// ---------------------------------------------------------------- prep
// h = hidden (zero-padded rows of ld), xg = h * gain0, the sum of squares of
// h per 16-column subtile, and the split A fragments of the first GEMM's
// input.  Work group (0, m) with m < the number of row tiles also clears
// the zero k-step of row tile m in both split buffers.
__device__ __forceinline__ void clear_zero_step(uint16_t* xs, int mt, int ks, int fpt, int lane) {
  uint4* f = reinterpret_cast<uint4*>(xs + ((size_t)mt * (ks + 1) + ks) * fpt * 512);
  for (int p = 0; p < fpt; ++p) f[p * 64 + lane] = make_uint4(0u, 0u, 0u, 0u);
}

__global__ void k_prep(float* h, float* xg, float* ss, int ss_ld, const float* hidden,
                       const float* gain0, int d, int ld, uint16_t* xs0, int ks0, uint16_t* xs1,
                       int ks1, bool stacked, bool two) {
  const int lane = threadIdx.x, g = blockIdx.x, m = blockIdx.y;
  const int n = g * kGroupCols + lane;
  const float v = n < d ? hidden[(size_t)m * d + n] : 0.f;
  h[(size_t)m * ld + n] = v;
  float x = v;
  if (gain0) {
    x = n < d ? v * gain0[n] : 0.f;
    xg[(size_t)m * ld + n] = x;
    const float sq = sum16(v * v);
    if ((lane & 15) == 0) ss[(size_t)m * ss_ld + g * 4 + (lane >> 4)] = sq;
  }
  if (xs0) {
    if (n < kKStep * ks0) xs_store(xs0, m, n, ks0, stacked, two, x);
    const int rpt = stacked ? kStackRows : 16, fpt = stacked ? 1 : 3;
    if (g == 0 && m * rpt < gridDim.y) {
      clear_zero_step(xs0, m, ks0, fpt, lane);
      if (xs1) clear_zero_step(xs1, m, ks1, fpt, lane);
    }
  }
}

hipError_t launch_prep(float* h, float* xg, float* ss, int ss_ld, const float* hidden,
                       const float* gain0, int M, int d, int ld, uint16_t* xs0, int ks0,
                       uint16_t* xs1, int ks1, bool two, hipStream_t st) {
  hipLaunchKernelGGL(k_prep, dim3(ld / kGroupCols, M), dim3(kWave), 0, st, h, xg, ss, ss_ld,
                     hidden, gain0, d, ld, xs0, ks0, xs1, ks1, xs_stacked(M), two);
  return hipGetLastError();
}

// ---------------------------------------------------------------- unit stats from given logits
// One 64-lane work group per (row, unit of four 16-column tiles).
__global__ void k_tile_stats(SampleArgs a) {
  const int r = blockIdx.y, lane = threadIdx.x, unit = blockIdx.x;
  const int n = unit * 4 * kSub + lane;
  const bool valid = n < a.V;
  const float l = valid ? a.logits[(size_t)r * a.ldl + n] : 0.f;
  const int b = r / (a.gamma + 1), i = r - b * (a.gamma + 1);
  const float qv = (valid && a.tmode != 0 && i < a.gamma)
                       ? a.q[((size_t)b * a.gamma + i) * a.V + n] : 0.f;
  lm_unit_stats(l, valid, true, n, r, unit, 4, a.G, a.gamma + 1, a.gamma, a.tmode, a.invT, qv,
                a.pst, a.pidx, a.qst);
}

hipError_t launch_tile_stats(const SampleArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_tile_stats, dim3(a.Gu, a.M), dim3(kWave), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- row stats
// One work group per row combines the row's G subtile statistics (G is
// even, so each 16-byte load carries two subtiles; padding subtiles hold
// neutral statistics).  Every thread issues its loads in batches of 8
// before merging, so a row costs one or two memory round trips.  T > 0:
// (max, 1 / Z) of p, or of q' for draft rows; T == 0: the argmax of p (in
// RI_M, as int bits).
constexpr int kRowThreads = 512;
constexpr int kRowBatch = 8;

__global__ __launch_bounds__(kRowThreads) void k_rowstats(SampleArgs a) {
  __shared__ float sh_m[kRowThreads / kWave], sh_s[kRowThreads / kWave];
  __shared__ int sh_i[kRowThreads / kWave];
  const int row = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool isq = row >= a.M;
  const size_t srow = isq ? (size_t)(row - a.M) : (size_t)row;
  const float4* st = reinterpret_cast<const float4*>((isq ? a.qst : a.pst) + srow * a.G * 2);
  const int2* sidx = reinterpret_cast<const int2*>(a.pidx + srow * a.G);
  const int n2 = a.G / 2;
  const bool greedy = a.tmode == 0;
  const bool plain_sum = isq && a.tmode == 1;
  const float it = isq ? 1.f : a.invT;
  float m = (plain_sum || greedy) ? (greedy ? -INFINITY : 0.f) : -INFINITY, s = 0.f;
  int idx = INT_MAX;
  for (int t0 = threadIdx.x; t0 < n2; t0 += kRowThreads * kRowBatch) {
    float4 v[kRowBatch];
    int2 ix[kRowBatch];
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u) {
      const int t = t0 + u * kRowThreads;
      v[u] = t < n2 ? st[t] : make_float4(-INFINITY, 0.f, -INFINITY, 0.f);
      if (greedy) ix[u] = t < n2 ? sidx[t] : make_int2(INT_MAX, INT_MAX);
      if (2 * t + 1 >= a.Gu) { v[u].z = -INFINITY; v[u].w = 0.f; ix[u].y = INT_MAX; }   // stride padding
    }
#pragma unroll
    for (int u = 0; u < kRowBatch; ++u) {
      if (greedy) {
        if (v[u].x > m || (v[u].x == m && ix[u].x < idx)) { m = v[u].x; idx = ix[u].x; }
        if (v[u].z > m || (v[u].z == m && ix[u].y < idx)) { m = v[u].z; idx = ix[u].y; }
      } else if (plain_sum) {
        s += v[u].y + v[u].w;
      } else {
        lse_merge(m, s, v[u].x, v[u].y, it);
        lse_merge(m, s, v[u].z, v[u].w, it);
      }
    }
  }
  if (greedy) wave_argmax(m, idx);
  else if (plain_sum) s = wave_sum(s);
  else wave_lse(m, s, it);
  if (lane == 0) { sh_m[wave] = m; sh_s[wave] = s; sh_i[wave] = idx; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float mm = sh_m[0], ss = sh_s[0];
    int ii = sh_i[0];
    for (int w = 1; w < kRowThreads / kWave; ++w) {
      if (greedy) {
        if (sh_m[w] > mm || (sh_m[w] == mm && sh_i[w] < ii)) { mm = sh_m[w]; ii = sh_i[w]; }
      } else if (plain_sum) {
        ss += sh_s[w];
      } else {
        lse_merge(mm, ss, sh_m[w], sh_s[w], it);
      }
    }
    float* ri = a.rowinfo + (size_t)row * kRowInfo;
    ri[RI_M] = greedy ? __int_as_float(ii) : mm;
    ri[RI_INVZ] = greedy ? 0.f : 1.0f / ss;
    ri[RI_THR] = 0.f;
    ri[RI_TIE] = 0.f;
    ri[RI_INVZN] = 1.0f;
    ri[RI_NUC] = 0.f;
  }
}

// ---------------------------------------------------------------- top-p
constexpr int kToppThreads = 1024;
constexpr int kToppWaves = kToppThreads / kWave;
constexpr int kHistCopies = 4;
constexpr int kMaxBins = 2048;           // digits of 11, 11 and 10 bits
// Histogram copies sit nb + 4 u64 apart (nb bins), so one bin of the four
// copies falls in four different LDS banks (a stride of nb alone is a
// multiple of the bank count, and the copies' lanes would conflict).
constexpr int kHistPad = 4;
constexpr int kToppBatch4 = 4;           // 16-byte loads of one batch (one or two batches in flight)
constexpr int kToppBatch1 = 8;           // 4-byte loads of one batch, rows that are not 16-byte aligned
constexpr int kTieCap = 64;              // tied keys ordered by one thread
constexpr int kCandPerWave = 512;        // candidate slots of each wave
typedef unsigned long long u64;

__device__ __forceinline__ u64 fixed_mass(float p) { return (u64)(p * 0x1.0p40f); }

// Exclusive prefix (thread order) of a u64 over the block; integer, so exact.
__device__ u64 block_excl_scan_u64(u64 x, u64* lds_waves) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  u64 inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const u64 y = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += y;
  }
  if (lane == 63) lds_waves[wave] = inc;
  __syncthreads();
  u64 base = 0;
  for (int w = 0; w < wave; ++w) base += lds_waves[w];
  __syncthreads();
  return base + inc - x;
}

struct ToppShared {
  // kHistCopies copies of the digit histogram, lane L adding to copy
  // L % kHistCopies, so lanes of a wave that share a digit collide at most
  // 64 / kHistCopies ways in the LDS atomic unit
  u64 hist[kHistCopies * (kMaxBins + kHistPad)];
  // The tokens of the first digit's crossing bucket (value bits, id), each
  // wave appending to its own segment during the second pass: they are the
  // only ones the last pass and the tie scan can match, so when they fit
  // those read LDS instead of the row.  Sums are integers, so the order of
  // the candidates changes no result.
  uint2 cand[kCandPerWave * kToppWaves];
  u64 tie_m[kTieCap];
  u64 lds_waves[kToppWaves];
  u64 above, total, zn;
  int tie_id[kTieCap];
  int ncw[kToppWaves];
  uint32_t prefix;
  int found, tie, nt, overflow;
};

// Nucleus of one row (p row, or draft row when ISQ): three radix passes
// over an order-preserving 32-bit key, 11, 11 and 10 bits, the first
// splitting each power-of-two range of values in four so that its
// crossing bucket is a small part of even a flat distribution.
// The row's (max, 1 / Z) from its unit statistics, as k_rowstats defines
// them (two block reductions: the max over the units' maxima, then the sum
// of s exp((m - max) / T); draft rows at T == 1 a plain sum), written to
// the row table with the no-nucleus defaults that a cut overwrites.  The
// top-p kernel does this for its row itself, one launch fewer.
template <bool ISQ>
__device__ __forceinline__ void topp_row_stats(const SampleArgs& a, int row, ToppShared& sh, float* ri,
                                               float& m_out, float& invz_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t srow = ISQ ? (size_t)(row - a.M) : (size_t)row;
  const float2* st = reinterpret_cast<const float2*>(ISQ ? a.qst : a.pst) + srow * a.G;
  const bool plain_sum = ISQ && a.tmode == 1;
  const float it = ISQ ? 1.f : a.invT;
  float* red = reinterpret_cast<float*>(sh.hist);   // scratch before the histograms
  float mx = -INFINITY;
  for (int t = tid; t < a.Gu; t += kToppThreads) {
    const float2 v = st[t];
    if (v.y > 0.f) mx = fmaxf(mx, v.x);
  }
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  float M = -INFINITY;
  for (int w = 0; w < kToppWaves; ++w) M = fmaxf(M, red[w]);
  float sum = 0.f;
  for (int t = tid; t < a.Gu; t += kToppThreads) {
    const float2 v = st[t];
    if (plain_sum) sum += v.y;
    else if (v.y > 0.f) sum += v.y * expf((v.x - M) * it);
  }
  sum = wave_sum(sum);
  if (lane == 0) red[kToppWaves + wave] = sum;
  __syncthreads();
  float S = 0.f;
  for (int w = 0; w < kToppWaves; ++w) S += red[kToppWaves + w];
  m_out = plain_sum ? 0.f : M;
  invz_out = 1.0f / S;
  if (tid == 0) {
    ri[RI_M] = m_out;
    ri[RI_INVZ] = invz_out;
    ri[RI_THR] = 0.f;
    ri[RI_TIE] = 0.f;
    ri[RI_INVZN] = 1.0f;
    ri[RI_NUC] = 0.f;
  }
  __syncthreads();   // the scratch becomes histograms
}

template <bool ISQ>
__device__ __forceinline__ void topp_row(const SampleArgs& a, int row, ToppShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float* ri = a.rowinfo + (size_t)row * kRowInfo;
  const float* src = ISQ ? a.q + (size_t)(row - a.M) * a.V : a.logits + (size_t)row * a.ldl;
  float m, invZ;
  topp_row_stats<ISQ>(a, row, sh, ri, m, invZ);
  const float invT = a.invT;
  const int tmode = a.tmode, V = a.V;

  // Masses only place the cut, so they use the hardware exp2 / log2: p rows
  // exp2((l - m) c) / Z with c = log2(e) / T; draft rows q / Z at T == 1,
  // else exp2(log2(q) / T - m log2(e)) / Z.
  constexpr float kLog2e = 1.4426950408889634f;
  const float c = invT * kLog2e, mq = m * kLog2e;
  auto key_of = [&](float x) -> uint32_t { return ISQ ? q_key(x) : logit_key(x); };
  auto mass_of = [&](float x) -> u64 {
    float p;
    if (!ISQ) p = __builtin_amdgcn_exp2f((x - m) * c) * invZ;
    else if (tmode == 1) p = x * invZ;
    else p = x > 0.f ? __builtin_amdgcn_exp2f(__builtin_amdgcn_logf(x) * invT - mq) * invZ : 0.f;
    return fixed_mass(p);
  };

  // Visits every token once.  Batches alternate between two register
  // buffers: batch k + 1 is issued into one before batch k is processed
  // from the other, and batch k + 2 before the wait for batch k + 1, so up
  // to two batches are in flight and no register copy waits on a load.
  // The loads are unconditional (a load past the row's end re-reads its
  // last element, whose token is skipped), so no branch separates a load
  // from its use; only the last batch checks bounds.  Rows that allow it
  // are read 16 bytes per lane (tokens 4 i .. 4 i + 3 of float4 i), else
  // 4 bytes per lane.
  const bool vec = (reinterpret_cast<uintptr_t>(src) & 15) == 0 && (V & 3) == 0;
  auto for_each_token = [&](auto&& f) {
    if (vec) {
      constexpr int B4 = kToppBatch4;
      constexpr int stride = B4 * kToppThreads;
      const float4* s4 = reinterpret_cast<const float4*>(src);
      const int V4 = V >> 2, last = V4 - 1;
      const int nbt = (V4 + stride - 1) / stride, nfull = V4 / stride;
      float4 ba[B4], bb[B4];
      auto issue = [&](float4 (&d)[B4], int bt) {
        const int i0 = tid + bt * stride;
#pragma unroll
        for (int u = 0; u < B4; ++u) d[u] = s4[min(i0 + u * kToppThreads, last)];
      };
      auto run = [&](const float4 (&d)[B4], int bt) {
        const int i0 = tid + bt * stride;
        const bool full = bt < nfull;
#pragma unroll
        for (int u = 0; u < B4; ++u) {
          const int i = i0 + u * kToppThreads;
          if (full || i < V4) {
            f(4 * i, d[u].x); f(4 * i + 1, d[u].y); f(4 * i + 2, d[u].z); f(4 * i + 3, d[u].w);
          }
        }
      };
      issue(ba, 0);
      for (int bt = 0; bt < nbt; bt += 2) {
        issue(bb, bt + 1);
        __builtin_amdgcn_sched_barrier(0);
        run(ba, bt);
        if (bt + 1 >= nbt) break;
        issue(ba, bt + 2);
        __builtin_amdgcn_sched_barrier(0);
        run(bb, bt + 1);
      }
      return;
    }
    constexpr int B1 = kToppBatch1;
    constexpr int stride = B1 * kToppThreads;
    const int nbt = (V + stride - 1) / stride, nfull = V / stride, last = V - 1;
    float ba[B1], bb[B1];
    auto issue = [&](float (&d)[B1], int bt) {
      const int v0 = tid + bt * stride;
#pragma unroll
      for (int u = 0; u < B1; ++u) d[u] = src[min(v0 + u * kToppThreads, last)];
    };
    auto run = [&](const float (&d)[B1], int bt) {
      const int v0 = tid + bt * stride;
      if (bt < nfull) {
#pragma unroll
        for (int u = 0; u < B1; ++u) f(v0 + u * kToppThreads, d[u]);
      } else {
#pragma unroll
        for (int u = 0; u < B1; ++u)
          if (v0 + u * kToppThreads < V) f(v0 + u * kToppThreads, d[u]);
      }
    };
    issue(ba, 0);
    for (int bt = 0; bt < nbt; bt += 2) {
      issue(bb, bt + 1);
      __builtin_amdgcn_sched_barrier(0);
      run(ba, bt);
      if (bt + 1 >= nbt) break;
      issue(ba, bt + 2);
      __builtin_amdgcn_sched_barrier(0);
      run(bb, bt + 1);
    }
  };
  // Candidates of this wave: segment cand[wave * kCandPerWave ...].
  uint2* wcand = sh.cand + wave * kCandPerWave;

  uint32_t prefix = 0, pmask = 0;
  u64 above = 0;
  double thr = 0.0;
  bool compact = false;
  for (int pass = 0; pass < 3; ++pass) {
    const int bits = pass < 2 ? 11 : 10;
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = 1 << bits;
    const int hs = nb + kHistPad;            // copy stride
    for (int i = tid; i < kHistCopies * hs; i += kToppThreads) sh.hist[i] = 0;
    if (tid == 0) sh.overflow = 0;
    __syncthreads();
    u64* myhist = sh.hist + (lane % kHistCopies) * hs;
    if (pass == 0) {
      for_each_token([&](int, float x) { atomicAdd(&myhist[key_of(x) >> 21], mass_of(x)); });
    } else if (pass == 1) {
      // The first digit's crossing bucket: its tokens are appended to the
      // wave's segment (a wave-uniform count, no atomics) in one pass over
      // the row that computes no mass, then the second digit's histogram
      // is taken over the candidates, every lane busy.  If any wave's
      // segment overflowed, the histogram takes a second pass over the row
      // instead (the same masses, so the same integer sums).
      const uint32_t p0 = prefix >> 21;
      int wn = 0;
      for_each_token([&](int v, float x) {
        const bool hit = (key_of(x) >> 21) == p0;
        const u64 mask = __ballot(hit);
        const int slot = wn + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
        if (hit && slot < kCandPerWave) wcand[slot] = make_uint2(__float_as_uint(x), (uint32_t)v);
        wn += __popcll(mask);
      });
      if (lane == 0) {
        sh.ncw[wave] = min(wn, kCandPerWave);
        if (wn > kCandPerWave) sh.overflow = 1;
      }
      __syncthreads();
      if (sh.overflow == 0) {
        const int n = min(wn, kCandPerWave);
        for (int i = lane; i < n; i += kWave) {
          const float x = __uint_as_float(wcand[i].x);
          atomicAdd(&myhist[(key_of(x) >> 10) & 2047u], mass_of(x));
        }
      } else {
        for_each_token([&](int, float x) {
          const uint32_t k = key_of(x);
          if ((k >> 21) == p0) atomicAdd(&myhist[(k >> 10) & 2047u], mass_of(x));
        });
      }
    } else if (compact) {
      const int n = sh.ncw[wave];
      for (int i = lane; i < n; i += kWave) {
        const float x = __uint_as_float(wcand[i].x);
        const uint32_t k = key_of(x);
        if ((k & pmask) == prefix) atomicAdd(&myhist[k & 1023u], mass_of(x));
      }
    } else {
      for_each_token([&](int, float x) {
        const uint32_t k = key_of(x);
        if ((k & pmask) == prefix) atomicAdd(&myhist[k & 1023u], mass_of(x));
      });
    }
    __syncthreads();
    if (pass == 1) compact = sh.overflow == 0;
    if (wave == 0) {
      // lane L holds bins [L bpl, (L + 1) bpl); masses of higher bins live in
      // higher lanes
      const int bpl = nb / kWave;
      auto bin = [&](int b) {
        u64 t = 0;
#pragma unroll
        for (int cc = 0; cc < kHistCopies; ++cc) t += sh.hist[cc * hs + b];
        return t;
      };
      // each lane's bins in a lane-rotated order, so that the lanes of a
      // step read different banks (integer sums: the order changes nothing)
      u64 S = 0;
      for (int j = 0; j < bpl; ++j) S += bin(lane * bpl + ((j + lane) & (bpl - 1)));
      u64 inc = S;   // inclusive suffix sum over lanes >= L
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const u64 y = __shfl_down(inc, o, kWave);
        if (lane + o < 64) inc += y;
      }
      if (pass == 0) {
        const u64 total = __shfl(inc, 0, kWave);
        if (lane == 0) sh.total = total;
        thr = (double)a.top_p * (double)total;
      }
      if (lane == 0) sh.found = 0;
      u64 cum = above + (inc - S);
      if ((double)cum < thr && (double)(cum + S) >= thr) {
        for (int j = bpl - 1; j >= 0; --j) {
          const u64 hj = bin(lane * bpl + j);
          if ((double)(cum + hj) >= thr) {
            sh.prefix = prefix | ((uint32_t)(lane * bpl + j) << shift);
            sh.above = cum;
            sh.found = 1;
            break;
          }
          cum += hj;
        }
      }
    }
    __syncthreads();
    if (pass == 0) thr = (double)a.top_p * (double)sh.total;
    if (!sh.found) return;   // no crossing (degenerate row): keep every token
    prefix = sh.prefix;
    pmask |= (uint32_t)(nb - 1) << shift;
    above = sh.above;
    __syncthreads();
  }

  // Tokens whose key equals the threshold key join in ascending id order.
  // They are gathered (id, mass); up to kTieCap of them are ordered by one
  // thread, more fall back to an ordered scan over per-thread id ranges.
  if (tid == 0) { sh.tie = INT_MAX; sh.nt = 0; }
  __syncthreads();
  auto gather_tie = [&](int v, float x) {
    if (key_of(x) == prefix) {
      const int slot = atomicAdd(&sh.nt, 1);
      if (slot < kTieCap) { sh.tie_id[slot] = v; sh.tie_m[slot] = mass_of(x); }
    }
  };
  if (compact) {
    const int n = sh.ncw[wave];
    for (int i = lane; i < n; i += kWave) gather_tie((int)wcand[i].y, __uint_as_float(wcand[i].x));
  } else {
    for_each_token(gather_tie);
  }
  __syncthreads();
  const int nt = sh.nt;
  if (nt <= kTieCap) {
    if (tid == 0) {
      // insertion sort by id, then the running mass in id order
      for (int i = 1; i < nt; ++i) {
        const int id = sh.tie_id[i];
        const u64 ms = sh.tie_m[i];
        int j = i - 1;
        while (j >= 0 && sh.tie_id[j] > id) { sh.tie_id[j + 1] = sh.tie_id[j]; sh.tie_m[j + 1] = sh.tie_m[j]; --j; }
        sh.tie_id[j + 1] = id;
        sh.tie_m[j + 1] = ms;
      }
      u64 cum = above;
      for (int i = 0; i < nt; ++i) {
        cum += sh.tie_m[i];
        if ((double)cum >= thr) { sh.tie = sh.tie_id[i]; sh.zn = cum; break; }
      }
    }
  } else {
    const int per = (V + kToppThreads - 1) / kToppThreads;
    const int v0 = min(V, tid * per), v1 = min(V, v0 + per);
    u64 local = 0;
    for (int v = v0; v < v1; ++v) {
      const float x = src[v];
      if (key_of(x) == prefix) local += mass_of(x);
    }
    const u64 excl = block_excl_scan_u64(local, sh.lds_waves);
    u64 cum = above + excl;
    for (int v = v0; v < v1; ++v) {
      const float x = src[v];
      if (key_of(x) != prefix) continue;
      cum += mass_of(x);
      if ((double)cum >= thr) {
        atomicMin(&sh.tie, v);
        break;
      }
    }
    __syncthreads();
    // the thread that owns the tie cut reports the nucleus mass
    const int tie = sh.tie;
    if (tie >= v0 && tie < v1 && tie != INT_MAX) sh.zn = cum;
  }
  __syncthreads();
  const int tie = sh.tie;
  if (tid == 0 && tie != INT_MAX) {
    ri[RI_THR] = __uint_as_float(prefix);
    ri[RI_TIE] = __int_as_float(tie);
    ri[RI_INVZN] = (float)((double)sh.total / (double)sh.zn);
    ri[RI_NUC] = __int_as_float(1);
  }
}

__global__ __launch_bounds__(kToppThreads) void k_topp(SampleArgs a) {
  __shared__ ToppShared sh;
  if ((int)blockIdx.x < a.M) topp_row<false>(a, blockIdx.x, sh);
  else topp_row<true>(a, blockIdx.x, sh);
}

// ---------------------------------------------------------------- resample helpers
// Token weights are fp32; every prefix sum of the inverse CDF is fp64, so
// the sampled token is not moved by summation error even when single
// tokens carry 1e-6 of the mass.
constexpr int kResThreads = 256;
constexpr int kResPer = kResampleChunk / kResThreads;   // contiguous ids per thread

// Inclusive scan over the wave in lane order.
__device__ __forceinline__ double wave_incl_scan_f64(double x) {
  const int lane = threadIdx.x & 63;
  double inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += y;
  }
  return inc;
}

// Exclusive scan over the wave in lane order; *total receives the wave sum.
__device__ __forceinline__ double wave_excl_scan_f64(double x, double* total) {
  const int lane = threadIdx.x & 63;
  const double inc = wave_incl_scan_f64(x);
  const double prev = __shfl_up(inc, 1, kWave);
  *total = __shfl(inc, 63, kWave);
  return lane == 0 ? 0.0 : prev;
}

// Block totals of x and y, each summed exactly as block_excl_scan_f64 sums
// its total (wave inclusive scans, then the waves in order), with one
// barrier for both.
__device__ void block_sum2_f64(double x, double y, double* lx, double* ly, double& tx, double& ty) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const double ix = wave_incl_scan_f64(x), iy = wave_incl_scan_f64(y);
  if (lane == 63) { lx[wave] = ix; ly[wave] = iy; }
  __syncthreads();
  double sx = 0.0, sy = 0.0;
  for (int w = 0; w < nw; ++w) { sx += lx[w]; sy += ly[w]; }
  tx = sx;
  ty = sy;
}

// Exclusive prefix over the block in thread order (wave scan, then waves in
// order); *total receives the block sum.
__device__ double block_excl_scan_f64(double x, double* lds_waves, double* total = nullptr) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const double inc = wave_incl_scan_f64(x);
  const double prev = __shfl_up(inc, 1, kWave);
  const double excl_lane = lane == 0 ? 0.0 : prev;
  if (lane == 63) lds_waves[wave] = inc;
  __syncthreads();
  double base = 0.0;
  for (int w = 0; w < wave; ++w) base += lds_waves[w];
  if (total) {
    double t = 0.0;
    for (int w = 0; w < nw; ++w) t += lds_waves[w];
    *total = t;
  }
  __syncthreads();
  return base + excl_lane;
}

// Weight of token v at the resample row: residual or p'.
struct ResRow {
  const float* l; const float* q; const float* rip; const float* riq;
  bool hasq; bool use_p; int tmode; float invT;
};
__device__ __forceinline__ float res_weight_lq(const ResRow& rr, int v, float l, float qv, float& pv) {
  pv = p_prime(rr.rip, l, v, rr.invT);
  if (!rr.hasq || rr.use_p) return pv;
  const float qq = q_prime(rr.riq, qv, v, rr.tmode, rr.invT);
  return fmaxf(pv - qq, 0.f);
}

// ri_seq: the sequence's row statistics in LDS (local rows: p rows 0..gamma,
// then the gamma q rows), else null for the global table.
__device__ __forceinline__ ResRow make_row(const SampleArgs& a, int b, int j, bool use_p,
                                           const float* ri_seq = nullptr) {
  const int G1 = a.gamma + 1;
  const size_t prow = (size_t)b * G1 + j;
  ResRow rr;
  rr.l = a.logits + prow * a.ldl;
  rr.rip = ri_seq ? ri_seq + j * kRowInfo : a.rowinfo + prow * kRowInfo;
  rr.hasq = j < a.gamma;
  const size_t qrow = (size_t)b * a.gamma + (rr.hasq ? j : 0);
  rr.q = a.q + qrow * a.V;
  rr.riq = ri_seq ? ri_seq + (G1 + (rr.hasq ? j : 0)) * kRowInfo
                  : a.rowinfo + ((size_t)a.M + qrow) * kRowInfo;
  rr.use_p = use_p;
  rr.tmode = a.tmode;
  rr.invT = a.invT;
  return rr;
}

// The kResPer contiguous logits and q values of this thread in chunk c
// (16-byte loads when the rows allow them).
__device__ __forceinline__ void load_chunk(const SampleArgs& a, const ResRow& rr, int c, float (&l)[kResPer],
                                           float (&qv)[kResPer]) {
  const int v0 = c * kResampleChunk + threadIdx.x * kResPer;
  const bool need_q = rr.hasq && !rr.use_p;
  const bool aligned = ((reinterpret_cast<uintptr_t>(rr.l + v0) |
                         (need_q ? reinterpret_cast<uintptr_t>(rr.q + v0) : 0)) & 15) == 0;
  if (v0 + kResPer <= a.V && aligned) {
    const float4 lv = *reinterpret_cast<const float4*>(rr.l + v0);
    l[0] = lv.x; l[1] = lv.y; l[2] = lv.z; l[3] = lv.w;
    if (need_q) {
      const float4 qq = *reinterpret_cast<const float4*>(rr.q + v0);
      qv[0] = qq.x; qv[1] = qq.y; qv[2] = qq.z; qv[3] = qq.w;
    } else {
#pragma unroll
      for (int e = 0; e < kResPer; ++e) qv[e] = 0.f;
    }
    return;
  }
#pragma unroll
  for (int e = 0; e < kResPer; ++e) {
    const int v = v0 + e;
    l[e] = v < a.V ? rr.l[v] : 0.f;
    qv[e] = (need_q && v < a.V) ? rr.q[v] : 0.f;
  }
}

// ---------------------------------------------------------------- decide + chunk sums
// Row statistics inside the decide kernel (no top-p, few short rows): every
// work group of sequence b merges the unit statistics of the sequence's
// 2 gamma + 1 rows itself, a wave per row, the same way in every group, so
// all groups hold the same bits; chunk 0 also writes them to the row table
// for the resample and the debug dumps.  This saves a launch and a memory
// round trip where the rows are short.
constexpr int kFuseRowsPerWave = 3;
constexpr int kFuseUnitsPerLane = 8;

bool fuse_rowstats(const SampleArgs& a, int threads) {
  return a.tmode != 0 && !(a.top_p < 1.0f) &&
         2 * a.gamma + 1 <= kFuseRowsPerWave * (threads / kWave) &&
         a.Gu <= kFuseUnitsPerLane * kWave;
}

// (max, 1 / Z) of the local rows of sequence b taken by this wave (rows
// wave, wave + nw, ...), as k_rowstats defines them, into ri_seq.  Two
// plain reductions per row instead of an online merge: the row max M over
// the units' maxima, then Z = sum over units of s * exp((m - M) / T).  The
// rows of a wave are reduced side by side.
__device__ void seq_rowstats(const SampleArgs& a, int b, float* ri_seq, bool publish) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int G1 = a.gamma + 1, nrows = 2 * a.gamma + 1;
  float2 v[kFuseRowsPerWave][kFuseUnitsPerLane];
  // every load first: one memory round trip for all of the wave's rows
#pragma unroll
  for (int k = 0; k < kFuseRowsPerWave; ++k) {
    const int r = min(wave + k * nw, nrows - 1);
    const bool isq = r >= G1;
    const size_t srow = isq ? (size_t)b * a.gamma + (r - G1) : (size_t)b * G1 + r;
    const float2* st = reinterpret_cast<const float2*>(isq ? a.qst : a.pst) + srow * a.G;
#pragma unroll
    for (int u = 0; u < kFuseUnitsPerLane; ++u) {
      const int t = lane + u * kWave;
      v[k][u] = t < a.Gu ? st[t] : make_float2(-INFINITY, 0.f);
    }
  }
  float mx[kFuseRowsPerWave], z[kFuseRowsPerWave];
#pragma unroll
  for (int k = 0; k < kFuseRowsPerWave; ++k) {
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < kFuseUnitsPerLane; ++u)
      if (v[k][u].y > 0.f) m = fmaxf(m, v[k][u].x);
    mx[k] = wave_max(m);
  }
#pragma unroll
  for (int k = 0; k < kFuseRowsPerWave; ++k) {
    const int r = min(wave + k * nw, nrows - 1);
    const bool isq = r >= G1;
    const bool plain_sum = isq && a.tmode == 1;
    const float it = isq ? 1.f : a.invT;
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < kFuseUnitsPerLane; ++u) {
      const float su = v[k][u].y;
      if (plain_sum) sum += su;
      else if (su > 0.f) sum += su * expf((v[k][u].x - mx[k]) * it);
    }
    z[k] = wave_sum(sum);
    if (plain_sum) mx[k] = 0.f;
  }
#pragma unroll
  for (int k = 0; k < kFuseRowsPerWave; ++k) {
    const int r = wave + k * nw;
    if (r < nrows && lane < kRowInfo) {
      float x = 0.f;
      if (lane == RI_M) x = mx[k];
      else if (lane == RI_INVZ) x = 1.0f / z[k];
      else if (lane == RI_INVZN) x = 1.0f;
      ri_seq[r * kRowInfo + lane] = x;
      if (publish) {
        const size_t grow = r >= G1 ? (size_t)a.M + (size_t)b * a.gamma + (r - G1) : (size_t)b * G1 + r;
        a.rowinfo[grow * kRowInfo + lane] = x;
      }
    }
  }
}

// Grid (chunks, B).  Every work group of sequence b takes the same decision
// (ratio test r * q'(x) < p'(x) per drafted position, first rejection;
// lattice-ai-eng explainer, acceptance rule; pigeon guide, How it works,
// step 3; at T = 0 the draft is compared to the argmax), chunk 0 writes
// it, and each work group then sums the weights of its 1024-token chunk of
// the resample row: the residual max(0, p' - q') at the first rejection,
// p' for the bonus slot, plus p' itself for a zero residual (pigeon guide,
// steps 4-5; scalablesystem article, The Accept/Reject Mechanism).
__global__ __launch_bounds__(kResThreads) void k_decide_chunks(SampleArgs a, bool fuse) {
  __shared__ int sh_bad, sh_first;
  __shared__ double lds_w[kResThreads / kWave], lds_p[kResThreads / kWave];
  __shared__ float sh_ri[kFuseRowsPerWave * (kResThreads / kWave) * kRowInfo];
  const int c = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int gamma = a.gamma, G1 = gamma + 1;
  if (tid == 0) { sh_bad = 0; sh_first = INT_MAX; }
  // this thread's draft token and the target / draft values at it, loaded
  // before the statistics (they need none)
  int x0 = -1;
  float l0 = 0.f, q0 = 0.f;
  if (tid < gamma) {
    x0 = a.draft[(size_t)b * gamma + tid];
    if (a.tmode != 0 && x0 >= 0 && x0 < a.V) {
      l0 = a.logits[((size_t)b * G1 + tid) * a.ldl + x0];
      q0 = a.q[((size_t)b * gamma + tid) * a.V + x0];
    }
  }
  if (fuse) seq_rowstats(a, b, sh_ri, c == 0);
  __syncthreads();
  // statistics of local row r (p rows 0..gamma, then q rows)
  auto ri_of = [&](int r) -> const float* {
    if (fuse) return sh_ri + r * kRowInfo;
    return a.rowinfo + (r < G1 ? (size_t)b * G1 + r : (size_t)a.M + (size_t)b * gamma + (r - G1)) * kRowInfo;
  };
  for (int i = tid; i < gamma; i += blockDim.x) {
    const int x = i == tid ? x0 : a.draft[(size_t)b * gamma + i];
    if (x < 0 || x >= a.V) { atomicOr(&sh_bad, 1); continue; }
    const size_t prow = (size_t)b * G1 + i;
    bool reject;
    if (a.tmode == 0) {
      reject = x != __float_as_int(ri_of(i)[RI_M]);
    } else {
      const size_t qrow = (size_t)b * gamma + i;
      const float lx = i == tid ? l0 : a.logits[prow * a.ldl + x];
      const float qx = i == tid ? q0 : a.q[qrow * a.V + x];
      const float pp = p_prime(ri_of(i), lx, x, a.invT);
      const float qq = q_prime(ri_of(G1 + i), qx, x, a.tmode, a.invT);
      float r;
      double u;
      row_uniforms(a.seed, b, i, r, u);
      reject = !(r * qq < pp);
    }
    if (reject) atomicMin(&sh_first, i);
  }
  __syncthreads();
  if (sh_bad) {
    if (c == 0) {
      for (int i = tid; i < G1; i += blockDim.x) a.emitted[(size_t)b * G1 + i] = -1;
      if (tid == 0) { a.n_acc[b] = -1; a.dec[4 * b] = -1; }
    }
    return;
  }
  const int n = min(sh_first, gamma);
  if (c == 0) {
    for (int i = tid; i < G1; i += blockDim.x) {
      int tok = -1;
      if (i < n) tok = a.draft[(size_t)b * gamma + i];
      else if (i == n && a.tmode == 0)
        tok = __float_as_int(ri_of(n)[RI_M]);
      a.emitted[(size_t)b * G1 + i] = tok;
    }
    if (tid == 0) { a.n_acc[b] = n; a.dec[4 * b] = n; }
  }
  if (a.tmode == 0) return;
  const ResRow rr = make_row(a, b, n, false, fuse ? sh_ri : nullptr);
  float l[kResPer], qv[kResPer];
  load_chunk(a, rr, c, l, qv);
  const int v0 = c * kResampleChunk + tid * kResPer;
  double sw = 0.0, sp = 0.0;
#pragma unroll
  for (int e = 0; e < kResPer; ++e) {
    if (v0 + e < a.V) {
      float pv;
      sw += (double)res_weight_lq(rr, v0 + e, l[e], qv[e], pv);
      sp += (double)pv;
    }
  }
  double tw, tp;
  block_sum2_f64(sw, sp, lds_w, lds_p, tw, tp);
  if (tid == 0) {
    a.csum[2 * ((size_t)b * a.nch + c)] = tw;
    a.csum[2 * ((size_t)b * a.nch + c) + 1] = tp;
  }
}

// ---------------------------------------------------------------- select
// Inverse CDF in token-id order: the chunk prefix is a block scan over the
// chunk sums; the chunk that crosses u * R is rescanned with the same
// per-thread weights, and the smallest id whose running fp64 prefix
// exceeds u * R is emitted.
__global__ __launch_bounds__(kResThreads) void k_res_select(SampleArgs a) {
  __shared__ double lds_w[kResThreads / kWave];
  __shared__ int sh_c, sh_cand, sh_last;
  __shared__ double sh_base, sh_lastbase;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const double* cs = a.csum + 2 * (size_t)b * a.nch;
  // The chunk sums do not depend on the decision: up to one per thread,
  // they load along with it.  Up to 64 chunks, every wave then scans them
  // itself (the same bits as the block scan, whose other waves would only
  // add zeros), with no LDS round trip or barrier.
  const bool one_wave = a.nch <= kWave;
  const int ci = one_wave ? lane : tid;
  double xw = 0.0, xp = 0.0;
  if (a.nch <= kResThreads && ci < a.nch) { xw = cs[2 * ci]; xp = cs[2 * ci + 1]; }
  const int j = a.dec[4 * b];
  if (j < 0) return;
  float r;
  double u;
  row_uniforms(a.seed, b, j, r, u);
  if (tid == 0) { sh_c = INT_MAX; sh_cand = INT_MAX; sh_last = -1; sh_base = 0.0; sh_lastbase = 0.0; }
  int usep = 0;
  double total = 0.0, target = 0.0;
  int c = 0;
  double base = 0.0;
  if (one_wave) {
    const bool in = lane < a.nch;
    double ex = wave_excl_scan_f64(xw, &total);
    if (!(total > 0.0)) {               // zero residual: sample p' instead
      usep = 1;
      xw = xp;
      ex = wave_excl_scan_f64(xw, &total);
    }
    target = u * total;
    const uint64_t over = __ballot(in && ex + xw > target);
    const uint64_t pos = __ballot(in && xw > 0.0);
    c = over ? __ffsll((unsigned long long)over) - 1 : (pos ? 63 - __clzll((unsigned long long)pos) : 0);
    base = __shfl(ex, c, kWave);
  } else if (a.nch <= kResThreads) {
    // one chunk sum per thread: one block scan picks the chunk
    const bool in = tid < a.nch;
    double ex = block_excl_scan_f64(xw, lds_w, &total);
    if (!(total > 0.0)) {               // zero residual: sample p' instead
      usep = 1;
      xw = xp;
      ex = block_excl_scan_f64(xw, lds_w, &total);
    }
    target = u * total;
    if (in && ex + xw > target) atomicMin(&sh_c, tid);
    if (in && xw > 0.0) atomicMax(&sh_last, tid);
    __syncthreads();
    const int pick = sh_c != INT_MAX ? sh_c : max(sh_last, 0);
    if (tid == pick) sh_base = ex;
    __syncthreads();
    if (tid == 0) { sh_c = pick; sh_last = -1; }
    __syncthreads();
    c = sh_c;
    base = sh_base;
  } else {
  // total of the residual chunk sums; the p' sums when it is exactly zero
  for (int pass = 0; pass < 2; ++pass) {
    total = 0.0;
    for (int c0 = 0; c0 < a.nch; c0 += kResThreads) {
      double t;
      const double x = c0 + tid < a.nch ? cs[2 * (c0 + tid) + pass] : 0.0;
      (void)block_excl_scan_f64(x, lds_w, &t);
      total += t;
    }
    usep = pass;
    if (total > 0.0) break;
  }
  target = u * total;
  // the first chunk whose inclusive prefix exceeds the target (the last
  // chunk when rounding leaves none)
  double run = 0.0;
  for (int c0 = 0; c0 < a.nch; c0 += kResThreads) {
    double t;
    const bool in = c0 + tid < a.nch;
    const double x = in ? cs[2 * (c0 + tid) + usep] : 0.0;
    const double ex = run + block_excl_scan_f64(x, lds_w, &t);
    if (in && ex + x > target) atomicMin(&sh_c, c0 + tid);
    if (c0 + tid == a.nch - 1) sh_lastbase = ex;
    __syncthreads();
    if (sh_c != INT_MAX) {
      if (c0 + tid == sh_c) sh_base = ex;
      break;
    }
    run += t;
  }
  __syncthreads();
  if (tid == 0 && sh_c == INT_MAX) { sh_c = a.nch - 1; sh_base = sh_lastbase; }
  __syncthreads();
  c = sh_c;
  base = sh_base;
  }
  const ResRow rr = make_row(a, b, j, usep != 0);
  float l[kResPer], qv[kResPer];
  load_chunk(a, rr, c, l, qv);
  const int v0 = c * kResampleChunk + tid * kResPer;
  float w[kResPer];
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < kResPer; ++e) {
    float pv;
    w[e] = v0 + e < a.V ? res_weight_lq(rr, v0 + e, l[e], qv[e], pv) : 0.f;
    s += (double)w[e];
  }
  const double E = block_excl_scan_f64(s, lds_w);
  double acc = 0.0;
  int cand = INT_MAX, last_pos = -1;
#pragma unroll
  for (int e = 0; e < kResPer; ++e) {
    const int v = v0 + e;
    if (v >= a.V || cand != INT_MAX) continue;
    acc += (double)w[e];
    if (w[e] > 0.f) last_pos = v;
    if (base + (E + acc) > target) cand = v;
  }
  cand = wave_min_int(cand);
  if ((tid & 63) == 0) atomicMin(&sh_cand, cand);
  atomicMax(&sh_last, last_pos);
  __syncthreads();
  // rounding can leave u*R past the rescanned chunk: take its last positive id
  const int tok = sh_cand != INT_MAX ? sh_cand : sh_last;
  if (tid == 0) a.emitted[(size_t)b * (a.gamma + 1) + j] = tok;
}

// ---------------------------------------------------------------- debug dumps
__global__ void k_dump_probs(SampleArgs a) {
  const int v = blockIdx.x * blockDim.x + threadIdx.x, row = blockIdx.y;
  if (v >= a.V) return;
  if (row < a.M) {
    if (a.p_out)
      a.p_out[(size_t)row * a.V + v] =
          p_prime(a.rowinfo + (size_t)row * kRowInfo, a.logits[(size_t)row * a.ldl + v], v, a.invT);
  } else if (a.q_out) {
    const size_t qrow = row - a.M;
    a.q_out[qrow * a.V + v] = q_prime(a.rowinfo + (size_t)row * kRowInfo, a.q[qrow * a.V + v], v,
                                      a.tmode, a.invT);
  }
}

hipError_t launch_dump_probs(const SampleArgs& a, hipStream_t st) {
  if (a.tmode == 0) return hipSuccess;
  hipLaunchKernelGGL(k_dump_probs, dim3((a.V + 255) / 256, a.M + a.B * a.gamma), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- tree walk
// Greedy verification of a draft tree ("Speculative Decoding: Speeding
// Sequential Generation", aicomputerinstitute.com, Tree-Based Drafting and
// Expected Tokens per Verification Round: Chain vs. Tree): one wave per
// sequence.  The pass scored the root row (local row 0) and one row per node
// (row 1 + j), whose argmax k_rowstats left in the row table.  From the
// root, the walk descends to the lowest-index child whose token equals the
// argmax of the current row, and stops at the first row none of whose
// children does, emitting that row's argmax.  Parents precede children
// (parent[j] < j), so every step moves to a higher node index and the walk
// ends within n + 1 steps.  A sequence with a parent outside [-1, j) or a
// token outside [0, V) gets n_accepted = -1 and all -1 outputs.
__global__ __launch_bounds__(kWave) void k_tree_walk(SampleArgs a, const int* parent,
                                                     const int* tokens, int* path) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int n = a.gamma, G1 = n + 1;
  const int* par = parent + (size_t)b * n;
  const int* tok = tokens + (size_t)b * n;
  int* em = a.emitted + (size_t)b * G1;
  int* pth = path ? path + (size_t)b * n : nullptr;
  bool bad = false;
  for (int j = lane; j < n; j += kWave) {
    const int pj = par[j], tj = tok[j];
    bad |= pj < -1 || pj >= j || tj < 0 || tj >= a.V;
  }
  if (__any(bad)) {
    for (int i = lane; i < G1; i += kWave) em[i] = -1;
    if (pth)
      for (int i = lane; i < n; i += kWave) pth[i] = -1;
    if (lane == 0) a.n_acc[b] = -1;
    return;
  }
  const float* ri = a.rowinfo + (size_t)b * G1 * kRowInfo;
  int cur = -1, depth = 0;
  for (int step = 0; step <= n; ++step) {
    const int am = __float_as_int(ri[(size_t)(cur + 1) * kRowInfo + RI_M]);
    int next = INT_MAX;
    for (int j0 = cur + 1; j0 < n; j0 += kWave) {   // children have higher indices
      const int j = j0 + lane;
      const bool hit = j < n && par[j] == cur && tok[j] == am;
      const uint64_t m = __ballot(hit);
      if (m) { next = j0 + __ffsll((unsigned long long)m) - 1; break; }
    }
    if (next == INT_MAX) {
      if (lane == 0) em[depth] = am;
      break;
    }
    if (lane == 0) {
      em[depth] = am;
      if (pth) pth[depth] = next;
    }
    ++depth;
    cur = next;
  }
  for (int i = depth + 1 + lane; i < G1; i += kWave) em[i] = -1;
  if (pth)
    for (int i = depth + lane; i < n; i += kWave) pth[i] = -1;
  if (lane == 0) a.n_acc[b] = depth;
}

hipError_t launch_tree_walk(const SampleArgs& a, const int* parent, const int* tokens, int* path,
                            hipStream_t st) {
  hipLaunchKernelGGL(k_rowstats, dim3(a.M), dim3(kRowThreads), 0, st, a);
  hipLaunchKernelGGL(k_tree_walk, dim3(a.B), dim3(kWave), 0, st, a, parent, tokens, path);
  return hipGetLastError();
}

// ---------------------------------------------------------------- sequencing
hipError_t launch_sampling(const SampleArgs& a, hipStream_t st) {
  const int qrows = a.B * a.gamma;
  const bool topp = a.tmode != 0 && a.top_p < 1.0f;
  const bool fuse = fuse_rowstats(a, kResThreads);
  // one work group per row combines the statistics, in parallel over rows
  // with top-p, the top-p kernel merges each row's statistics itself
  if (!fuse && !topp)
    hipLaunchKernelGGL(k_rowstats, dim3(a.tmode != 0 ? a.M + qrows : a.M), dim3(kRowThreads), 0, st, a);
  if (topp) hipLaunchKernelGGL(k_topp, dim3(a.M + qrows), dim3(kToppThreads), 0, st, a);
  hipLaunchKernelGGL(k_decide_chunks, dim3(a.tmode != 0 ? a.nch : 1, a.B), dim3(kResThreads), 0, st, a,
                     fuse);
  if (a.tmode != 0)
    hipLaunchKernelGGL(k_res_select, dim3(a.B), dim3(kResThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace sv
