// Attention of a verification pass's new rows over a KV-cached prefix, and
// the commit of the accepted rows ("Speculative Decoding: Speeding Sequential
// Generation", aicomputerinstitute.com, Constructing the Tree Attention Mask
// in Code; "Build a Speculative Decoding Engine to Cut LLM Latency by 3x",
// scalablesystem.dev, KV Cache Management for Dual Models, Rollback
// Protocol).
//
// Cache layout, bf16: keys [B][Hkv][max_seq][HD] (one key's head dimension
// is a contiguous row), values [B][Hkv][HD][max_seq] (head-dimension major:
// eight consecutive positions of one dimension are 16 contiguous bytes, the
// B operand of the P V product).  New row i of sequence b is the query
// q[b][i][h][:] (fp32); its key and value sit at slot L_b + i.  Row i sees
// slots 0 .. L_b - 1 and the new slots of itself and its ancestors.
//
// Work decomposition: a work group owns (sequence, KV head, group of up to
// 128 query rows: new rows x the H / Hkv query heads sharing the KV head,
// split of the keys); each of its waves owns one 16-row tile of those rows,
// and the group stages each 64-key tile of keys and values in LDS once for
// all of them, so every key and value byte of a split is read from memory
// once for all query rows of the group (the weight-streaming idea of the
// GEMMs, applied to the cache).  Both products run on bf16 MFMA (16x16x32):
// a wave's queries are split once into three bf16 terms (exact) and held as
// B fragments in registers; the products are taken transposed (S^T = K Q^T,
// O^T = V^T P^T, keys and values as A operands from LDS), so the scores'
// softmax runs on the accumulators with each lane owning one query row (16
// of its 64 scores of a key tile in registers, the rest in three other
// lanes); the probabilities go through LDS into the operand layout, split
// into two terms (2^-16 relative).  Online softmax per row; every wave
// writes its rows' partial (max, sum, unnormalised output) for the split,
// and a second kernel merges the splits' partials in a fixed order, so
// results are run-to-run identical (with one split the output is written
// directly).  The softmax runs in base 2: the queries are multiplied by
// scale * log2(e) (one fp32 rounding) before they are split, so the
// accumulators hold scores in log2 units and a probability is the hardware
// exp2 of a difference (about one ulp), with no multiply per score; the
// running maxima and the partials' maxima are in the same units.  Both
// errors are far below the score error of an fp32 128-term dot product that
// bounds the output.

#include <algorithm>
#include <climits>
#include <cmath>
#include <type_traits>

#include "common.h"
#include "internal.h"
#include "specverify.h"

#pragma clang fp contract(off)

namespace sv {

constexpr int kAttnMaxRT = 8;      // 16-row tiles of query rows per work group (at most)
constexpr int kAttnTile = 64;      // keys per tile: four 16-key MFMA tiles
constexpr float kAttnSlack = 11.5f;  // a row's reference max moves when passed by more (2^11.5 ~ 3e3)
#ifndef SV_ATTN_WAVES
#define SV_ATTN_WAVES 2048         // waves a launch aims for (splits of the keys): two per SIMD
#endif
#ifndef SV_ATTN_MIN_TILES
#define SV_ATTN_MIN_TILES 4        // fewest 64-key tiles per split
#endif
constexpr int kAttnMaxSplits = 256;  // splits of the keys (LDS of the combine)

struct AttnArgs {
  int B, n_new, H, Hkv, G, max_seq, R, RG, S;   // R = n_new * G rows, RG row groups, S splits
  const float* q;            // [B][n_new][H][HD]
  const uint16_t* k;         // [B][Hkv][max_seq][HD]
  const uint16_t* vt;        // [B][Hkv][HD][max_seq]  (values, head-dimension major)
  const int* cache_len;      // [B]
  const int* parent;         // [B][n_new] or null (chain)
  float scale;
  float* part_o;             // [B][Hkv][RG][S][16 RT][HD]
  float* part_ml;            // [B][Hkv][RG][S][16 RT][2]
  float* out;                // [B][n_new][H][HD]
};

__device__ __forceinline__ int attn_len(const AttnArgs& a, int b) {
  // committed length, clamped so the new slots stay inside the cache
  const int L = a.cache_len[b];
  return L < 0 ? 0 : (L > a.max_seq - a.n_new ? a.max_seq - a.n_new : L);
}

// Eight fp32 values as three bf16 A/B fragments (hi, mid, lo): exact, so a
// bf16 MFMA over the three reproduces an fp32 product up to accumulation.
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8 (&f)[3]) {
  uint32_t t[3][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t a0, b0, c0, a1, b1, c1;
    split3_bf16(x[2 * j], a0, b0, c0);
    split3_bf16(x[2 * j + 1], a1, b1, c1);
    t[0][j] = a0 | (a1 << 16);
    t[1][j] = b0 | (b1 << 16);
    t[2][j] = c0 | (c1 << 16);
  }
#pragma unroll
  for (int p = 0; p < 3; ++p) {
    const u32x4 u = {t[p][0], t[p][1], t[p][2], t[p][3]};
    f[p] = __builtin_bit_cast(bf16x8, u);
  }
}

// Eight fp32 values in [0, 1] as two bf16 fragments (hi, lo by truncation):
// |x - hi - lo| <= 2^-16 |x|, for the softmax probabilities.
__device__ __forceinline__ void split8_2(const float (&x)[8], bf16x8 (&f)[2]) {
  uint32_t t[2][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t h0 = __float_as_uint(x[2 * j]) & 0xffff0000u;
    const uint32_t h1 = __float_as_uint(x[2 * j + 1]) & 0xffff0000u;
    const uint32_t l0 = __float_as_uint(x[2 * j] - __uint_as_float(h0)) >> 16;
    const uint32_t l1 = __float_as_uint(x[2 * j + 1] - __uint_as_float(h1)) >> 16;
    t[0][j] = (h0 >> 16) | h1;
    t[1][j] = l0 | (l1 << 16);
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const u32x4 u = {t[p][0], t[p][1], t[p][2], t[p][3]};
    f[p] = __builtin_bit_cast(bf16x8, u);
  }
}

// Zero the bf16 values of a fragment whose keys (first key k0, eight in a
// row) are at or past `end`: memory past the visible keys may hold anything.
__device__ __forceinline__ bf16x8 zero_past(bf16x8 f, int k0, int end) {
  if (k0 + 8 <= end) return f;
  u32x4 u = __builtin_bit_cast(u32x4, f);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t w = u[j];
    if (k0 + 2 * j >= end) w &= 0xffff0000u;
    if (k0 + 2 * j + 1 >= end) w &= 0x0000ffffu;
    u[j] = w;
  }
  return __builtin_bit_cast(bf16x8, u);
}

// Each wave owns one 16-row tile of the group's query rows and streams every
// key tile of the split; the group stages each 64-key tile of keys and
// values in LDS once for all its waves (loaded through registers a tile
// ahead, stored between two barriers).  A wave holds one row tile's
// accumulators (under 190 registers), so two waves share a SIMD: two
// four-wave groups per CU up to 64 rows, one eight-wave group up to 128.
// Each wave's state is final for its rows over the split: no merge across
// waves.  Tiles in LDS are padded (keys HD + 8, values 64 + 8 bf16 per row)
// so the 16-byte operand reads of a wave fall in distinct bank groups.
template <int RT>
struct AttnGroupWaves { static constexpr int value = RT <= 4 ? 4 : 8; };

template <int HD, int RT>
__global__ __launch_bounds__(64 * AttnGroupWaves<RT>::value) void k_decode_attn(AttnArgs a) {
  constexpr int NW = AttnGroupWaves<RT>::value, THREADS = 64 * NW;
  constexpr int KS = HD / 32;                      // 32-dimension k-steps of a score
  constexpr int DT = HD / 16;                      // 16-dimension output tiles
  constexpr int ROWS = 16 * RT;
  constexpr int KLD = HD + 8, VLD = kAttnTile + 8; // LDS row strides (bf16)
  constexpr int KPR = HD / 8, VPR = kAttnTile / 8; // 16-byte chunks per key / value row
  constexpr int KPT = kAttnTile * KPR / THREADS, VPT = HD * VPR / THREADS;
  static_assert(KPT * THREADS == kAttnTile * KPR && VPT * THREADS == HD * VPR,
                "whole 16-byte chunks per thread");
  __shared__ uint64_t anc[64];
  __shared__ __align__(16) uint16_t kl[kAttnTile * KLD];
  __shared__ __align__(16) uint16_t vl[HD * VLD];
  __shared__ __align__(16) float pbuf[NW][16][kAttnTile + 4];
  const int lane = threadIdx.x & 63, tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.x, rg = blockIdx.y % a.RG, kvh = blockIdx.y / a.RG, b = blockIdx.z;
  const int L = attn_len(a, b), T = L + a.n_new;
  const int r0 = rg * ROWS, nr = min(ROWS, a.R - r0);
  const int g = lane >> 4, c = lane & 15;          // C layout: rows 4 g + j, column c
  const bool live = wave < RT;                     // waves past the row tiles only load

  if (tid == 0) {
    uint64_t m = 0;
    for (int i = 0; i < a.n_new; ++i) {
      int p = a.parent ? a.parent[(size_t)b * a.n_new + i] : i - 1;
      if (p < -1 || p >= i) p = -1;                // a bad parent sees no other new row
      m = (p >= 0 ? anc[p] : 0ull) | (1ull << i);
      anc[i] = m;
    }
  }
  // this lane's query row (16 wave + c) as B fragments: dimensions
  // 32 ks + 8 g .. + 7, times scale * log2(e), in three exact bf16 terms
  const int r = wave * 16 + c;
  const int rowi = live && r < nr ? (r0 + r) / a.G : -1;
  bf16x8 qf[KS][3];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    float v[8];
    if (rowi >= 0) {
      const int rr = r0 + r, h = kvh * a.G + rr % a.G;
      const float4* qp = reinterpret_cast<const float4*>(
          a.q + (((size_t)b * a.n_new + rowi) * a.H + h) * HD + ks * 32 + 8 * g);
      const float4 u0 = qp[0], u1 = qp[1];
      const float qs = a.scale * 1.44269504088896341f;   // scale * log2(e)
      v[0] = u0.x * qs; v[1] = u0.y * qs; v[2] = u0.z * qs; v[3] = u0.w * qs;
      v[4] = u1.x * qs; v[5] = u1.y * qs; v[6] = u1.z * qs; v[7] = u1.w * qs;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = 0.f;
    }
    split8(v, qf[ks]);
  }
  __syncthreads();

  // this group's keys: split `split` of S, in 64-key tiles
  const int per_split = (((T + a.S - 1) / a.S) + kAttnTile - 1) / kAttnTile * kAttnTile;
  const int s0 = min(T, split * per_split), s1 = min(T, s0 + per_split);
  const uint16_t* K = a.k + ((size_t)b * a.Hkv + kvh) * a.max_seq * HD;
  const uint16_t* Vt = a.vt + ((size_t)b * a.Hkv + kvh) * (size_t)HD * a.max_seq;

  // tile loads: chunk x of the keys is key x / KPR, dimensions 8 (x % KPR);
  // of the values, dimension x / VPR, keys 8 (x % VPR).  Keys past the
  // split read its last key; values past it are zeroed when stored.
  bf16x8 kr[KPT], vr[VPT];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int x = tid + i * THREADS, key = min(t + x / KPR, s1 - 1);
      kr[i] = *reinterpret_cast<const bf16x8*>(K + (size_t)key * HD + 8 * (x % KPR));
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int x = tid + i * THREADS;
      const int k0 = min(t + 8 * (x % VPR), a.max_seq - 8);   // in bounds: max_seq % 8 == 0
      vr[i] = *reinterpret_cast<const bf16x8*>(Vt + (size_t)(x / VPR) * a.max_seq + k0);
    }
  };
  auto store_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int x = tid + i * THREADS;
      *reinterpret_cast<bf16x8*>(&kl[(x / KPR) * KLD + 8 * (x % KPR)]) = kr[i];
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int x = tid + i * THREADS;
      *reinterpret_cast<bf16x8*>(&vl[(x / VPR) * VLD + 8 * (x % VPR)]) =
          zero_past(vr[i], t + 8 * (x % VPR), s1);
    }
  };

  float m = -INFINITY, l = 0.f;
  f32x4 acc_o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc_o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint64_t vis_new = rowi >= 0 ? anc[rowi] : 0ull;
  if (s0 < s1) load_tile(s0);
  for (int t = s0; t < s1; t += kAttnTile) {
    __syncthreads();                                 // the last tile's reads are done
    store_tile(t);
    __syncthreads();                                 // this tile is in LDS
    if (t + kAttnTile < s1) load_tile(t + kAttnTile);
    if (!live) continue;
    // scores S^T[key][row] of the four 16-key tiles
    f32x4 acc_s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) acc_s[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 kf[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        kf[kt] = *reinterpret_cast<const bf16x8*>(&kl[(16 * kt + c) * KLD + 32 * ks + 8 * g]);
#pragma unroll
      for (int p = 0; p < 3; ++p)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
          acc_s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kt], qf[ks][p], acc_s[kt], 0, 0, 0);
    }
    // mask and online softmax of the lane's row (as in k_decode_attn)
    const bool plain = t + kAttnTile <= min(L, s1);
    float mt = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bool vis = rowi >= 0;
        if (!plain) {
          const int key = t + 16 * kt + 4 * g + j, jn = key - L;
          vis = vis && key < s1 && (jn < 0 || ((vis_new >> jn) & 1ull));
        }
        acc_s[kt][j] = vis ? acc_s[kt][j] : -INFINITY;
        mt = fmaxf(mt, acc_s[kt][j]);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 16, kWave));
    mt = fmaxf(mt, __shfl_xor(mt, 32, kWave));
    const float mn = m == -INFINITY || mt > m + kAttnSlack ? fmaxf(m, mt) : m;
    const float mref = mn > -INFINITY ? mn : 0.f;
    float ps = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      float4 pv;
      pv.x = __builtin_amdgcn_exp2f(acc_s[kt][0] - mref);
      pv.y = __builtin_amdgcn_exp2f(acc_s[kt][1] - mref);
      pv.z = __builtin_amdgcn_exp2f(acc_s[kt][2] - mref);
      pv.w = __builtin_amdgcn_exp2f(acc_s[kt][3] - mref);
      ps += (pv.x + pv.y) + (pv.z + pv.w);
      *reinterpret_cast<float4*>(&pbuf[wave][c][16 * kt + 4 * g]) = pv;
    }
    ps += __shfl_xor(ps, 16, kWave);
    ps += __shfl_xor(ps, 32, kWave);
    float cr = 1.f;
    bool moved = false;
    if (mn > m) {
      cr = m > -INFINITY ? __builtin_amdgcn_exp2f(m - mn) : 0.f;
      moved = true;
    }
    l = l * cr + ps;
    m = mn;
    if (t != s0 && __any(moved)) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc_o[dt][j] *= cr;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // O^T += V^T P^T, P in two bf16 terms (2^-16 relative)
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      const float4* pp = reinterpret_cast<const float4*>(&pbuf[wave][c][32 * kv + 8 * g]);
      const float4 u0 = pp[0], u1 = pp[1];
      const float x[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
      bf16x8 pf[2];
      split8_2(x, pf);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(&vl[(16 * dt + c) * VLD + 32 * kv + 8 * g]);
#pragma unroll
        for (int p = 0; p < 2; ++p)
          acc_o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[p], acc_o[dt], 0, 0, 0);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  // the rows' states over this split: lane (g, c) holds row r at dimensions
  // 16 dt + 4 g + j; with one split, the output o / l itself
  if (!live || r >= nr) return;
  if (a.S == 1) {
    const int rr = r0 + r, h = kvh * a.G + rr % a.G;
    float* out = a.out + (((size_t)b * a.n_new + rowi) * a.H + h) * HD;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) out[16 * dt + 4 * g + j] = l > 0.f ? acc_o[dt][j] / l : 0.f;
    return;
  }
  const size_t unit = (((size_t)b * a.Hkv + kvh) * a.RG + rg) * (size_t)a.S + split;
  float* po = a.part_o + (unit * ROWS + r) * HD;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    *reinterpret_cast<float4*>(&po[16 * dt + 4 * g]) =
        make_float4(acc_o[dt][0], acc_o[dt][1], acc_o[dt][2], acc_o[dt][3]);
  if (g == 0) {
    a.part_ml[(unit * ROWS + r) * 2] = m;
    a.part_ml[(unit * ROWS + r) * 2 + 1] = l;
  }
}

// Merge the S partial states of every query row in order: out =
// sum_p o_p 2^(m_p - M) / sum_p l_p 2^(m_p - M), M the largest m_p (maxima
// in log2 units).
// kCombineRows rows per work group, one thread per (row, dimension) or per
// (row, four dimensions).  The
// splits' (m, l) pairs are read once, in parallel, into LDS, and their
// weights computed there, so the loads of a row's S partial outputs do not
// depend on one another and stay in flight together; the sums still run in
// split order.  Every split writes its partial (an empty one: o = 0,
// m = -inf, l = 0), so a weight of 0 adds exactly 0.  Launched only when
// S > 1; with one split the attention writes the output itself.
constexpr int kCombineRows = 4;
template <int HD, int DPT>
__global__ __launch_bounds__(HD / DPT * kCombineRows) void k_attn_combine(AttnArgs a, int rows) {
  static_assert(DPT == 1 || DPT == 4, "one or four dimensions per thread");
  constexpr int TR = HD / DPT;                   // threads per row
  __shared__ float wsh[kCombineRows][kAttnMaxSplits], lsh[kCombineRows][kAttnMaxSplits];
  const int dq = threadIdx.x % TR, cr = threadIdx.x / TR;
  const int r = blockIdx.x * kCombineRows + cr, rg = blockIdx.y % a.RG, kvh = blockIdx.y / a.RG,
            b = blockIdx.z;
  const int rr = rg * rows + r;
  const bool live = r < rows && rr < a.R;        // every thread reaches the barriers
  const int P = a.S;
  const size_t unit0 = (((size_t)b * a.Hkv + kvh) * a.RG + rg) * (size_t)P;
  if (live) {
    for (int p = dq; p < P; p += TR) {
      wsh[cr][p] = a.part_ml[((unit0 + p) * rows + r) * 2];
      lsh[cr][p] = a.part_ml[((unit0 + p) * rows + r) * 2 + 1];
    }
  }
  __syncthreads();
  float M = -INFINITY;
  if (live)
    for (int p = 0; p < P; ++p) M = fmaxf(M, wsh[cr][p]);
  __syncthreads();
  if (live) {
    for (int p = dq; p < P; p += TR) {
      const float mp = wsh[cr][p];
      wsh[cr][p] = M > -INFINITY && mp > -INFINITY ? __builtin_amdgcn_exp2f(mp - M) : 0.f;
    }
  }
  __syncthreads();
  if (!live) return;
  float den = 0.f;
  for (int p = 0; p < P; ++p) den += lsh[cr][p] * wsh[cr][p];
  // the partial rows sit in the workspace (256-byte aligned): with four
  // dimensions per thread, 16-byte loads
  using V = typename std::conditional<DPT == 4, float4, float>::type;
  const V* po = reinterpret_cast<const V*>(a.part_o + unit0 * rows * HD + (size_t)r * HD) + dq;
  const size_t step = (size_t)rows * TR;
  float num[DPT];
#pragma unroll
  for (int e = 0; e < DPT; ++e) num[e] = 0.f;
  auto add = [&](const V& o, float w) {
    if constexpr (DPT == 4) {
      num[0] += o.x * w; num[1] += o.y * w; num[2] += o.z * w; num[3] += o.w * w;
    } else {
      num[0] += o * w;
    }
  };
  int p = 0;
  for (; p + 8 <= P; p += 8) {
    V o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = po[(p + j) * step];
#pragma unroll
    for (int j = 0; j < 8; ++j) add(o[j], wsh[cr][p + j]);
  }
  for (; p < P; ++p) add(po[p * step], wsh[cr][p]);
  const int i = rr / a.G, h = kvh * a.G + rr % a.G;
  float* out = a.out + (((size_t)b * a.n_new + i) * a.H + h) * HD + DPT * dq;
#pragma unroll
  for (int e = 0; e < DPT; ++e) out[e] = den > 0.f ? num[e] / den : 0.f;
}

// ---------------------------------------------------------------- commit
// Tree commit: the accepted path's rows (node j = new row j + 1) gathered to
// slots L + 1 .. L + n, for every KV head: key rows ([slot][HD]) and value
// columns ([HD][slot]); everything is read before anything is written.  One
// work group per (KV head, sequence).
template <int HD>
__global__ __launch_bounds__(256) void k_kv_gather(int B, int n_new, int Hkv, int max_seq,
                                                   uint16_t* k, uint16_t* vt, const int* cache_len,
                                                   const int* n_accepted, const int* path) {
  __shared__ uint32_t krows[64][HD / 2];
  __shared__ uint16_t vcols[64][HD];
  const int kvh = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int n = n_accepted[b];
  if (n <= 0 || n > n_new - 1) return;
  int L = cache_len[b];
  L = L < 0 ? 0 : (L > max_seq - n_new ? max_seq - n_new : L);
  const size_t base = ((size_t)b * Hkv + kvh) * max_seq * HD;
  uint32_t* K32 = reinterpret_cast<uint32_t*>(k + base);
  uint16_t* VT = vt + base;
  constexpr int W = HD / 2;
  auto node_of = [&](int kk) {
    const int node = path[(size_t)b * (n_new - 1) + kk];
    return node < 0 ? 0 : (node > n_new - 2 ? n_new - 2 : node);
  };
  for (int x = tid; x < n * W; x += 256) {
    const int kk = x / W, cc = x - kk * W;
    krows[kk][cc] = K32[(size_t)(L + 1 + node_of(kk)) * W + cc];
  }
  for (int x = tid; x < n * HD; x += 256) {
    const int kk = x % n, d = x / n;
    vcols[kk][d] = VT[(size_t)d * max_seq + L + 1 + node_of(kk)];
  }
  __syncthreads();
  for (int x = tid; x < n * W; x += 256) {
    const int kk = x / W, cc = x - kk * W;
    K32[(size_t)(L + 1 + kk) * W + cc] = krows[kk][cc];
  }
  for (int x = tid; x < n * HD; x += 256) {
    const int kk = x % n, d = x / n;
    VT[(size_t)d * max_seq + L + 1 + kk] = vcols[kk][d];
  }
}

// The pointer move of a commit (after any gather, on the same stream).
__global__ void k_kv_advance(int B, const int* n_accepted, int* cache_len) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B && n_accepted[b] >= 0) cache_len[b] += n_accepted[b] + 1;
}

}  // namespace sv

using namespace sv;

namespace {

struct AttnShape {
  int R = 0, RT = 0, RG = 0, S = 0;
  size_t o_off = 0, ml_off = 0, total = 0;
};

AttnShape attn_shape(int B, int n_new, int H, int Hkv, int hd, int max_seq) {
  AttnShape s;
  const int G = H / Hkv;
  s.R = n_new * G;
  // row tiles per work group: all rows in one group up to 128 (every key and
  // value byte read once for them), else groups of 128
  s.RT = std::min(kAttnMaxRT, (s.R + 15) / 16);
  s.RG = (s.R + 16 * s.RT - 1) / (16 * s.RT);
  // splits of the keys: about SV_ATTN_WAVES waves over the chip (two per
  // SIMD: 1024 and 4096 measured slower, and 1536 and 3072 as well, on
  // B = 4 tree rows), but at least SV_ATTN_MIN_TILES 64-key tiles per split
  // (four: B = 1, 8192 keys 22.4 -> 21.1 us against one, fewer partials to
  // merge; two changed nothing)
  const int groups = B * Hkv * s.RG;
  const int tiles = (max_seq + kAttnTile - 1) / kAttnTile;
  const int nw = s.RT <= 4 ? 4 : 8;                 // waves of a group (AttnGroupWaves)
  const int want = (SV_ATTN_WAVES + groups * nw - 1) / (groups * nw);
  const int most = std::max(1, tiles / SV_ATTN_MIN_TILES);
  s.S = std::max(1, std::min(std::min(want, most), kAttnMaxSplits));
  const size_t units = (size_t)groups * s.S;
  const size_t rows = (size_t)16 * s.RT;
  s.o_off = 0;
  s.ml_off = (units * rows * hd * sizeof(float) + 255) & ~(size_t)255;
  s.total = s.ml_off + ((units * rows * 2 * sizeof(float) + 255) & ~(size_t)255);
  return s;
}

bool attn_args_ok(int B, int n_new, int H, int Hkv, int hd, int max_seq) {
  return B >= 1 && n_new >= 1 && n_new <= 64 && Hkv >= 1 && H >= Hkv && H % Hkv == 0 &&
         (hd == 64 || hd == 128) && max_seq >= n_new && max_seq >= 8 && max_seq % 8 == 0;
}

}  // namespace

extern "C" {

size_t spec_attention_workspace_size(int32_t B, int32_t n_new, int32_t H, int32_t Hkv,
                                     int32_t head_dim, int32_t max_seq) {
  if (!attn_args_ok(B, n_new, H, Hkv, head_dim, max_seq)) return 0;
  return attn_shape(B, n_new, H, Hkv, head_dim, max_seq).total;
}

spec_status spec_decode_attention(int32_t B, int32_t n_new, int32_t H, int32_t Hkv,
                                  int32_t head_dim, int32_t max_seq, const float* q,
                                  const uint16_t* k_cache, const uint16_t* v_cache,
                                  const int32_t* cache_len, const int32_t* parent, float scale,
                                  float* out, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  if (!attn_args_ok(B, n_new, H, Hkv, head_dim, max_seq) || !q || !k_cache || !v_cache ||
      !cache_len || !out || !(scale > 0.f) || !std::isfinite(scale))
    return SPEC_EINVAL;
  if ((reinterpret_cast<uintptr_t>(k_cache) & 15) || (reinterpret_cast<uintptr_t>(v_cache) & 15))
    return SPEC_EINVAL;
  const AttnShape s = attn_shape(B, n_new, H, Hkv, head_dim, max_seq);
  if (!workspace || workspace_bytes < s.total || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return SPEC_EWORKSPACE;
  AttnArgs a;
  a.B = B; a.n_new = n_new; a.H = H; a.Hkv = Hkv; a.G = H / Hkv; a.max_seq = max_seq;
  a.R = s.R; a.RG = s.RG; a.S = s.S;
  a.q = q; a.k = k_cache; a.vt = v_cache; a.cache_len = cache_len; a.parent = parent;
  a.scale = scale; a.out = out;
  a.part_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + s.o_off);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + s.ml_off);
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const dim3 grid(s.S, Hkv * s.RG, B), cgrid(16 * s.RT / kCombineRows, Hkv * s.RG, B);
  auto go = [&](auto hd_tag, auto rt_tag) {
    constexpr int HDc = decltype(hd_tag)::value, RTc = decltype(rt_tag)::value;
    hipLaunchKernelGGL((k_decode_attn<HDc, RTc>), grid, dim3(64 * AttnGroupWaves<RTc>::value), 0, st, a);
    // few splits: four dimensions per thread (fewer, fuller work groups);
    // many: one, so more loads of a row's partials are in flight at once
    if (s.S > 16)
      hipLaunchKernelGGL((k_attn_combine<HDc, 1>), cgrid, dim3(HDc * kCombineRows), 0, st, a, 16 * RTc);
    else if (s.S > 1)
      hipLaunchKernelGGL((k_attn_combine<HDc, 4>), cgrid, dim3(HDc / 4 * kCombineRows), 0, st, a, 16 * RTc);
  };
  auto by_rt = [&](auto hd_tag) {
    switch (s.RT) {
      case 1: go(hd_tag, std::integral_constant<int, 1>{}); break;
      case 2: go(hd_tag, std::integral_constant<int, 2>{}); break;
      case 3: go(hd_tag, std::integral_constant<int, 3>{}); break;
      case 4: go(hd_tag, std::integral_constant<int, 4>{}); break;
      case 5: go(hd_tag, std::integral_constant<int, 5>{}); break;
      case 6: go(hd_tag, std::integral_constant<int, 6>{}); break;
      case 7: go(hd_tag, std::integral_constant<int, 7>{}); break;
      default: go(hd_tag, std::integral_constant<int, 8>{}); break;
    }
  };
  if (head_dim == 128) by_rt(std::integral_constant<int, 128>{});
  else by_rt(std::integral_constant<int, 64>{});
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

spec_status spec_kv_commit(int32_t B, int32_t n_new, int32_t Hkv, int32_t head_dim,
                           int32_t max_seq, uint16_t* k_cache, uint16_t* v_cache,
                           int32_t* cache_len, const int32_t* n_accepted, const int32_t* path,
                           void* stream) {
  if (B < 1 || n_new < 1 || n_new > 64 || Hkv < 1 || (head_dim != 64 && head_dim != 128) ||
      max_seq < n_new || !cache_len || !n_accepted)
    return SPEC_EINVAL;
  if (path && (!k_cache || !v_cache || (reinterpret_cast<uintptr_t>(k_cache) & 3) ||
               (reinterpret_cast<uintptr_t>(v_cache) & 3)))
    return SPEC_EINVAL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (path && n_new > 1) {
    if (max_seq % 8) return SPEC_EINVAL;
    if (head_dim == 128)
      hipLaunchKernelGGL(k_kv_gather<128>, dim3(Hkv, B), dim3(256), 0, st, B, n_new, Hkv, max_seq,
                         k_cache, v_cache, cache_len, n_accepted, path);
    else
      hipLaunchKernelGGL(k_kv_gather<64>, dim3(Hkv, B), dim3(256), 0, st, B, n_new, Hkv, max_seq,
                         k_cache, v_cache, cache_len, n_accepted, path);
  }
  hipLaunchKernelGGL(k_kv_advance, dim3((B + 255) / 256), dim3(256), 0, st, B, n_accepted, cache_len);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

}  // extern "C"
