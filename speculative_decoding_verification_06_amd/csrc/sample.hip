// The acceptance rule over the vocabulary, after the target pass.
//
//   rowstats : combine per-tile (max, sum exp) of each logits row into
//              softmax(l / T), and the per-tile sums of each draft row into
//              q' = q^(1/T) / sum ("Speculative decoding" pigeon guide, When it
//              breaks: the same temperature / top-p on p and q)
//   topp     : nucleus of each row by an 8-bit-digit radix select on an
//              order-preserving key, with masses in 2^-40 fixed point so the
//              histogram sums are exact and order independent
//   decide   : ratio test r * q'(x) < p'(x) per drafted position, first
//              rejection per sequence (lattice-ai-eng explainer, acceptance
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
// input.  Work group (0, m) with m < ceil(M / 16) also clears the zero
// k-step of row tile m in both split buffers.
__device__ __forceinline__ void clear_zero_step(uint16_t* xs, int mt, int ks, int lane) {
  uint4* f = reinterpret_cast<uint4*>(xs + ((size_t)mt * (ks + 1) + ks) * 3 * 512);
#pragma unroll
  for (int p = 0; p < 3; ++p) f[p * 64 + lane] = make_uint4(0u, 0u, 0u, 0u);
}

__global__ void k_prep(float* h, float* xg, float* ss, int ss_ld, const float* hidden,
                       const float* gain0, int d, int ld, uint16_t* xs0, int ks0, uint16_t* xs1,
                       int ks1) {
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
    if (n < kKStep * ks0) xs_store(xs0, m, n, ks0, x);
    if (g == 0 && m * 16 < gridDim.y) {
      clear_zero_step(xs0, m, ks0, lane);
      if (xs1) clear_zero_step(xs1, m, ks1, lane);
    }
  }
}

hipError_t launch_prep(float* h, float* xg, float* ss, int ss_ld, const float* hidden,
                       const float* gain0, int M, int d, int ld, uint16_t* xs0, int ks0,
                       uint16_t* xs1, int ks1, hipStream_t st) {
  hipLaunchKernelGGL(k_prep, dim3(ld / kGroupCols, M), dim3(kWave), 0, st, h, xg, ss, ss_ld,
                     hidden, gain0, d, ld, xs0, ks0, xs1, ks1);
  return hipGetLastError();
}

// ---------------------------------------------------------------- subtile stats from given logits
__global__ void k_tile_stats(SampleArgs a) {
  const int r = blockIdx.y, lane = threadIdx.x;
  const int tile = blockIdx.x * 4 + (lane >> 4);
  const int n = tile * kSub + (lane & 15);
  const bool live = tile < a.G;
  const bool valid = live && n < a.V;
  const float l = valid ? a.logits[(size_t)r * a.ldl + n] : 0.f;
  lm_subtile_stats(l, valid, live, n, r, tile, a.G, a.gamma + 1, a.gamma, a.V, a.tmode, a.invT,
                   a.q, a.pst, a.pidx, a.qst);
}

hipError_t launch_tile_stats(const SampleArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_tile_stats, dim3((a.G + 3) / 4, a.M), dim3(kWave), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- row stats
constexpr int kRowThreads = 256;

__global__ __launch_bounds__(kRowThreads) void k_rowstats(SampleArgs a) {
  __shared__ float sh_m[kRowThreads / kWave], sh_s[kRowThreads / kWave];
  const int row = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool isq = row >= a.M;
  const float* st = isq ? a.qst + (size_t)(row - a.M) * a.G * 2 : a.pst + (size_t)row * a.G * 2;
  const bool plain_sum = isq && a.tmode == 1;
  const float it = isq ? 1.f : a.invT;
  float m = plain_sum ? 0.f : -INFINITY, s = 0.f;
  for (int t = threadIdx.x; t < a.G; t += kRowThreads) {
    if (plain_sum) s += st[2 * t + 1];
    else lse_merge(m, s, st[2 * t], st[2 * t + 1], it);
  }
  if (plain_sum) s = wave_sum(s);
  else wave_lse(m, s, it);
  if (lane == 0) { sh_m[wave] = m; sh_s[wave] = s; }
  __syncthreads();
  if (threadIdx.x == 0) {
    float mm = sh_m[0], ss = sh_s[0];
    for (int w = 1; w < kRowThreads / kWave; ++w) {
      if (plain_sum) ss += sh_s[w];
      else lse_merge(mm, ss, sh_m[w], sh_s[w], it);
    }
    float* ri = a.rowinfo + (size_t)row * kRowInfo;
    ri[RI_M] = mm;
    ri[RI_INVZ] = 1.0f / ss;
    ri[RI_THR] = 0.f;
    ri[RI_TIE] = 0.f;
    ri[RI_INVZN] = 1.0f;
    ri[RI_NUC] = 0.f;
  }
}

// ---------------------------------------------------------------- top-p
constexpr int kToppThreads = 1024;
typedef unsigned long long u64;

__device__ __forceinline__ u64 fixed_mass(float p) { return (u64)(p * 0x1.0p40f); }

// Exclusive prefix (thread order) of a u64 over the block; integer, so exact.
__device__ u64 block_excl_scan_u64(u64 x, u64* lds_waves) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
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
  (void)nw;
  __syncthreads();
  return base + inc - x;
}

__global__ __launch_bounds__(kToppThreads) void k_topp(SampleArgs a) {
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool isq = row >= a.M;
  float* ri = a.rowinfo + (size_t)row * kRowInfo;
  const float* src = isq ? a.q + (size_t)(row - a.M) * a.V : a.logits + (size_t)row * a.ldl;
  const float m = ri[RI_M], invZ = ri[RI_INVZ], invT = a.invT;
  const int tmode = a.tmode, V = a.V;

  __shared__ u64 hist[256];
  __shared__ u64 sh_above, sh_total, sh_zn;
  __shared__ uint32_t sh_prefix;
  __shared__ int sh_found, sh_tie;
  __shared__ u64 lds_waves[kToppThreads / 64];

  auto key_of = [&](float x) -> uint32_t { return isq ? q_key(x) : logit_key(x); };
  auto mass_of = [&](float x) -> u64 {
    const float p = isq ? q_tempered(ri, x, tmode, invT) : expf((x - m) * invT) * invZ;
    return fixed_mass(p);
  };

  uint32_t prefix = 0, pmask = 0;
  u64 above = 0;
  double thr = 0.0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += kToppThreads) hist[i] = 0;
    __syncthreads();
    for (int v = tid; v < V; v += kToppThreads) {
      const float x = src[v];
      const uint32_t k = key_of(x);
      if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], mass_of(x));
    }
    __syncthreads();
    if (wave == 0) {
      // lane L holds bins 4L..4L+3; masses of higher bins live in higher lanes
      u64 h[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) h[j] = hist[4 * lane + j];
      const u64 S = h[0] + h[1] + h[2] + h[3];
      u64 inc = S;   // inclusive suffix sum over lanes >= L
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const u64 y = __shfl_down(inc, o, kWave);
        if (lane + o < 64) inc += y;
      }
      if (pass == 0) {
        const u64 total = __shfl(inc, 0, kWave);
        if (lane == 0) sh_total = total;
        thr = (double)a.top_p * (double)total;
      }
      if (lane == 0) sh_found = 0;
      u64 cum = above + (inc - S);
      if ((double)cum < thr && (double)(cum + S) >= thr) {
#pragma unroll
        for (int j = 3; j >= 0; --j) {
          if ((double)(cum + h[j]) >= thr) {
            sh_prefix = prefix | ((uint32_t)(4 * lane + j) << shift);
            sh_above = cum;
            sh_found = 1;
            break;
          }
          cum += h[j];
        }
      }
    }
    __syncthreads();
    if (pass == 0) thr = (double)a.top_p * (double)sh_total;
    if (!sh_found) return;   // no crossing (degenerate row): keep every token
    prefix = sh_prefix;
    pmask |= 0xffu << shift;
    above = sh_above;
    __syncthreads();
  }

  // Tokens whose key equals the threshold key join in ascending id order.
  const int per = (V + kToppThreads - 1) / kToppThreads;
  const int v0 = min(V, tid * per), v1 = min(V, v0 + per);
  u64 local = 0;
  for (int v = v0; v < v1; ++v) {
    const float x = src[v];
    if (key_of(x) == prefix) local += mass_of(x);
  }
  if (tid == 0) sh_tie = INT_MAX;
  const u64 excl = block_excl_scan_u64(local, lds_waves);
  u64 cum = above + excl;
  for (int v = v0; v < v1; ++v) {
    const float x = src[v];
    if (key_of(x) != prefix) continue;
    cum += mass_of(x);
    if ((double)cum >= thr) {
      atomicMin(&sh_tie, v);
      break;
    }
  }
  __syncthreads();
  // the thread that owns the tie cut reports the nucleus mass
  const int tie = sh_tie;
  if (tie >= v0 && tie < v1 && tie != INT_MAX) sh_zn = cum;
  __syncthreads();
  if (tid == 0 && tie != INT_MAX) {
    ri[RI_THR] = __uint_as_float(prefix);
    ri[RI_TIE] = __int_as_float(tie);
    ri[RI_INVZN] = (float)((double)sh_total / (double)sh_zn);
    ri[RI_NUC] = __int_as_float(1);
  }
}

// ---------------------------------------------------------------- decide
__global__ void k_decide(SampleArgs a) {
  extern __shared__ int sh_am[];          // [gamma + 1] argmax per row (greedy)
  __shared__ int sh_bad, sh_first;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gamma = a.gamma, G1 = gamma + 1;
  if (tid == 0) { sh_bad = 0; sh_first = INT_MAX; }
  __syncthreads();
  for (int i = tid; i < gamma; i += blockDim.x) {
    const int x = a.draft[(size_t)b * gamma + i];
    if (x < 0 || x >= a.V) atomicOr(&sh_bad, 1);
  }
  __syncthreads();
  if (sh_bad) {
    for (int i = tid; i < G1; i += blockDim.x) a.emitted[(size_t)b * G1 + i] = -1;
    if (tid == 0) { a.n_acc[b] = -1; a.dec[4 * b] = -1; }
    return;
  }
  int first = INT_MAX;
  if (a.tmode == 0) {
    for (int i = wave; i < G1; i += blockDim.x / kWave) {
      const size_t row = (size_t)b * G1 + i;
      float v = -INFINITY;
      int idx = INT_MAX;
      for (int t = lane; t < a.G; t += kWave) {
        const float tv = a.pst[2 * (row * a.G + t)];
        const int ti = a.pidx[row * a.G + t];
        if (tv > v || (tv == v && ti < idx)) { v = tv; idx = ti; }
      }
      wave_argmax(v, idx);
      if (lane == 0) sh_am[i] = idx;
    }
    __syncthreads();
    for (int i = tid; i < gamma; i += blockDim.x)
      if (a.draft[(size_t)b * gamma + i] != sh_am[i]) first = min(first, i);
  } else {
    for (int i = tid; i < gamma; i += blockDim.x) {
      const int x = a.draft[(size_t)b * gamma + i];
      const size_t prow = (size_t)b * G1 + i, qrow = (size_t)b * gamma + i;
      const float pp = p_prime(a.rowinfo + prow * kRowInfo, a.logits[prow * a.ldl + x], x, a.invT);
      const float qq = q_prime(a.rowinfo + ((size_t)a.M + qrow) * kRowInfo, a.q[qrow * a.V + x],
                               x, a.tmode, a.invT);
      float r, u;
      row_uniforms(a.seed, b, i, r, u);
      if (!(r * qq < pp)) first = min(first, i);
    }
  }
  first = wave_min_int(first);
  if (lane == 0) atomicMin(&sh_first, first);
  __syncthreads();
  const int n = min(sh_first, gamma);
  for (int i = tid; i < G1; i += blockDim.x) {
    int tok = -1;
    if (i < n) tok = a.draft[(size_t)b * gamma + i];
    else if (i == n && a.tmode == 0) tok = sh_am[n];
    a.emitted[(size_t)b * G1 + i] = tok;
  }
  if (tid == 0) { a.n_acc[b] = n; a.dec[4 * b] = n; }
}

// ---------------------------------------------------------------- resample
// Token weights are fp32; every prefix sum of the inverse CDF is fp64, so
// the sampled token is not moved by summation error even when single
// tokens carry 1e-6 of the mass.
constexpr int kResThreads = 256;
constexpr int kResPer = kResampleChunk / kResThreads;   // contiguous ids per thread

// Exclusive prefix over the block in thread order (wave scan, then waves in order).
__device__ double block_excl_scan_f64(double x, double* lds_waves) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += y;
  }
  const double prev = __shfl_up(inc, 1, kWave);
  const double excl_lane = lane == 0 ? 0.0 : prev;
  if (lane == 63) lds_waves[wave] = inc;
  __syncthreads();
  double base = 0.0;
  for (int w = 0; w < wave; ++w) base += lds_waves[w];
  __syncthreads();
  return base + excl_lane;
}

// Weight of token v at the resample row: residual or p'.
struct ResRow {
  const float* l; const float* q; const float* rip; const float* riq;
  bool hasq; bool use_p; int tmode; float invT;
};
__device__ __forceinline__ float res_weight(const ResRow& rr, int v, float& pv) {
  pv = p_prime(rr.rip, rr.l[v], v, rr.invT);
  if (!rr.hasq || rr.use_p) return pv;
  const float qv = q_prime(rr.riq, rr.q[v], v, rr.tmode, rr.invT);
  return fmaxf(pv - qv, 0.f);
}

__device__ __forceinline__ ResRow make_row(const SampleArgs& a, int b, int j, bool use_p) {
  const int G1 = a.gamma + 1;
  const size_t prow = (size_t)b * G1 + j;
  ResRow rr;
  rr.l = a.logits + prow * a.ldl;
  rr.rip = a.rowinfo + prow * kRowInfo;
  rr.hasq = j < a.gamma;
  const size_t qrow = (size_t)b * a.gamma + (rr.hasq ? j : 0);
  rr.q = a.q + qrow * a.V;
  rr.riq = a.rowinfo + ((size_t)a.M + qrow) * kRowInfo;
  rr.use_p = use_p;
  rr.tmode = a.tmode;
  rr.invT = a.invT;
  return rr;
}

__global__ __launch_bounds__(kResThreads) void k_res_chunks(SampleArgs a) {
  __shared__ double lds_w[4], lds_p[4];
  const int c = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int j = a.dec[4 * b];
  if (j < 0) return;
  const ResRow rr = make_row(a, b, j, false);
  double sw = 0.0, sp = 0.0;
  const int v0 = c * kResampleChunk + tid * kResPer;
  for (int e = 0; e < kResPer; ++e) {
    const int v = v0 + e;
    if (v < a.V) {
      float pv;
      sw += (double)res_weight(rr, v, pv);
      sp += (double)pv;
    }
  }
  const double ew = block_excl_scan_f64(sw, lds_w);
  const double ep = block_excl_scan_f64(sp, lds_p);
  if (tid == kResThreads - 1) {
    a.csum[2 * ((size_t)b * a.nch + c)] = ew + sw;
    a.csum[2 * ((size_t)b * a.nch + c) + 1] = ep + sp;
  }
}

__global__ __launch_bounds__(kResThreads) void k_res_select(SampleArgs a) {
  extern __shared__ double sh_C[];         // [nch] running chunk prefix
  __shared__ double lds_w[4];
  __shared__ int sh_c, sh_usep, sh_cand, sh_last;
  __shared__ double sh_base, sh_t;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int j = a.dec[4 * b];
  if (j < 0) return;
  // chunk sums into LDS in parallel ([0, nch) residual, [nch, 2 nch) p'),
  // then one thread forms the running prefix in chunk order
  const double* cs = a.csum + 2 * (size_t)b * a.nch;
  for (int c = tid; c < a.nch; c += kResThreads) {
    sh_C[c] = cs[2 * c];
    sh_C[a.nch + c] = cs[2 * c + 1];
  }
  __syncthreads();
  if (tid == 0) {
    double C = 0.0;
    for (int c = 0; c < a.nch; ++c) { C = C + sh_C[c]; sh_C[c] = C; }
    int usep = 0;
    if (!(C > 0.0)) {
      usep = 1;
      C = 0.0;
      for (int c = 0; c < a.nch; ++c) { C = C + sh_C[a.nch + c]; sh_C[c] = C; }
    }
    float r, u;
    row_uniforms(a.seed, b, j, r, u);
    const double t = (double)u * C;
    int cs_ = a.nch - 1;
    for (int c = 0; c < a.nch; ++c)
      if (sh_C[c] > t) { cs_ = c; break; }
    sh_c = cs_;
    sh_base = cs_ > 0 ? sh_C[cs_ - 1] : 0.0;
    sh_t = t;
    sh_usep = usep;
    sh_cand = INT_MAX;
    sh_last = -1;
  }
  __syncthreads();
  const ResRow rr = make_row(a, b, j, sh_usep != 0);
  const int v0 = sh_c * kResampleChunk + tid * kResPer;
  double s = 0.0;
  for (int e = 0; e < kResPer; ++e) {
    const int v = v0 + e;
    if (v < a.V) { float pv; s += (double)res_weight(rr, v, pv); }
  }
  const double E = block_excl_scan_f64(s, lds_w);
  const double base = sh_base, t = sh_t;
  double run = 0.0;
  int cand = INT_MAX, last_pos = -1;
  for (int e = 0; e < kResPer; ++e) {
    const int v = v0 + e;
    if (v >= a.V) break;
    float pv;
    const float w = res_weight(rr, v, pv);
    run += (double)w;
    if (w > 0.f) last_pos = v;
    if (base + (E + run) > t) { cand = v; break; }
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

// ---------------------------------------------------------------- sequencing
hipError_t launch_sampling(const SampleArgs& a, hipStream_t st) {
  const int qrows = a.B * a.gamma;
  if (a.tmode != 0) {
    hipLaunchKernelGGL(k_rowstats, dim3(a.M + qrows), dim3(kRowThreads), 0, st, a);
    if (a.top_p < 1.0f)
      hipLaunchKernelGGL(k_topp, dim3(a.M + qrows), dim3(kToppThreads), 0, st, a);
  }
  hipLaunchKernelGGL(k_decide, dim3(a.B), dim3(256), (a.gamma + 1) * sizeof(int), st, a);
  if (a.tmode != 0) {
    hipLaunchKernelGGL(k_res_chunks, dim3(a.nch, a.B), dim3(kResThreads), 0, st, a);
    hipLaunchKernelGGL(k_res_select, dim3(a.B), dim3(kResThreads), 2 * a.nch * sizeof(double), st, a);
  }
  return hipGetLastError();
}

}  // namespace sv
