// Device helpers shared by the gfx950 kernels of the verification step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace sv {

constexpr int kWave = 64;
constexpr int kGroupCols = 64;     // columns of one packed weight block (4 MFMA tiles)
constexpr int kSub = 16;           // columns of one MFMA tile = one statistics subtile
constexpr int kKStep = 32;         // K rows per MFMA step (16x16x32)

// ---- bfloat16 ------------------------------------------------------------
// A bf16 is the top half of an fp32, so widening is a shift.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round fp32 to bf16, nearest-even (finite inputs).
__device__ __forceinline__ uint32_t bf16_bits_rne(float x) {
  uint32_t b = __float_as_uint(x);
  b += 0x7fffu + ((b >> 16) & 1u);
  return b >> 16;
}

// Exact split of an fp32 value into three bf16 terms, x = hi + mid + lo, by
// truncation: hi keeps the top 8 significant bits, x - hi is exact in fp32
// and holds at most 16 significant bits, mid keeps its top 8, and the rest
// (at most 8 bits) is a bf16 exactly.  The three products with a bf16
// weight are therefore exact, and an MFMA over the three terms reproduces
// an fp32 x fp32 dot product up to the accumulation rounding.
__device__ __forceinline__ void split3_bf16(float x, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  const uint32_t b0 = __float_as_uint(x) & 0xffff0000u;
  const float r1 = x - __uint_as_float(b0);
  const uint32_t b1 = __float_as_uint(r1) & 0xffff0000u;
  const float r2 = r1 - __uint_as_float(b1);
  hi = b0 >> 16;
  mid = b1 >> 16;
  lo = __float_as_uint(r2) >> 16;
}

// Two-term split, both terms rounded to nearest even: |x - hi| <= 2^-8 |x|,
// so x - hi is exact in fp32 (hi lies within a factor of two of x), and
// lo = bf16(x - hi) leaves |x - hi - lo| <= 2^-16 |x|.  Finite x only.
__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b + 0x7fffu + ((b >> 16) & 1u)) & 0xffff0000u;
}
__device__ __forceinline__ void split2_bf16(float x, uint32_t& hi, uint32_t& lo) {
  const uint32_t b0 = bf16_rne_bits(x);
  hi = b0 >> 16;
  lo = bf16_rne_bits(x - __uint_as_float(b0)) >> 16;
}

// Split activations in MFMA A-operand order.  For a GEMM input X[M][K]
// with KS k-steps of 32 (step KS is all zero), one 1 KiB fragment holds 64
// lanes x 8 bf16, lane L holding A-rows L % 16 at columns
// 32 s + 8 (L / 16) + j of k-step s.  Packings:
//   plain   : row tile mt = 16 rows; k-step s of the tile is three
//             fragments (hi, mid, lo), all multiplied into one accumulator;
//             with the two-term split the third fragment is not written, and
//             every GEMM of such a pass reads two fragments per row tile (the
//             all-zero k-step past the end holds zeros in all three)
//   stacked : one fragment per k-step whose A-row R p + r holds term p of
//             row R mt + r, so a single MFMA covers every term of R rows and
//             the terms are summed after the k-loop: R = kStackRows = 5 rows
//             of three terms (A-row 15 unused), or, with the two-term split,
//             R = kStackRows2 = 8 rows of two terms
// xs_index returns the bf16 index of term 0 of (row, col); term p sits at
// +p * xs_term_step(stacked, two).  Both are host functions too, so the
// host-side access check evaluates the very formulas the kernels use.
constexpr int kStackRows = 5;
constexpr int kStackRows2 = 8;
__host__ __device__ __forceinline__ int xs_stack_rows(bool two) { return two ? kStackRows2 : kStackRows; }
__host__ __device__ __forceinline__ int xs_term_step(bool stacked, bool two) {
  return stacked ? 8 * xs_stack_rows(two) : 512;
}
__host__ __device__ __forceinline__ size_t xs_index(int row, int col, int ks, bool stacked, bool two) {
  const int lane_hi = 16 * ((col & 31) >> 3), s = col >> 5, j = col & 7;
  if (stacked) {
    const int R = xs_stack_rows(two);
    const size_t frag = (size_t)(row / R) * (ks + 1) + s;
    return (frag * 64 + lane_hi + row % R) * 8 + j;
  }
  const size_t frag = ((size_t)(row >> 4) * (ks + 1) + s) * 3;
  return (frag * 64 + lane_hi + (row & 15)) * 8 + j;
}
__device__ __forceinline__ void xs_store(uint16_t* xs, int row, int col, int ks, bool stacked,
                                         bool two, float x) {
  uint32_t a, b, c = 0;
  if (two) split2_bf16(x, a, b);
  else split3_bf16(x, a, b, c);
  const size_t i = xs_index(row, col, ks, stacked, two);
  const int st = xs_term_step(stacked, two);
  xs[i] = (uint16_t)a;
  xs[i + st] = (uint16_t)b;
  if (!two) xs[i + 2 * st] = (uint16_t)c;
}

// ---- Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11) -------------------
// Each round: (hi0,lo0) = M0*c0, (hi1,lo1) = M1*c2,
// c = (hi1^c1^k0, lo1, hi0^c3^k1, lo0); the key is bumped by the Weyl
// constants between rounds.
__device__ __forceinline__ void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += W0; k1 += W1; }
    const uint64_t hi0 = __umul64hi(M0, c[0]), lo0 = M0 * c[0];
    const uint64_t hi1 = __umul64hi(M1, c[2]), lo1 = M1 * c[2];
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
  }
}

// Uniforms of batch row b, position i: word 0 -> r (ratio test), its top 24
// bits scaled by 2^-24, exact in fp32 where the test runs; word 1 -> u
// (inverse CDF), its top 53 bits scaled by 2^-53, exact in fp64 where u * R
// is formed, so the sampled law is not rounded to steps of 2^-24.
__device__ __forceinline__ void row_uniforms(uint64_t seed, int b, int i, float& r, double& u) {
  uint64_t c[4] = {(uint64_t)i, (uint64_t)b, 0ull, 0ull};
  philox4x64_10(c, seed, 0ull);
  r = (float)(uint32_t)(c[0] >> 40) * 0x1.0p-24f;
  u = (double)(c[1] >> 11) * 0x1.0p-53;
}

// ---- cross-lane steps ------------------------------------------------------
// A 16-lane group is one DPP row, so the butterfly runs on row rotations
// (VALU operands, no trip through the LDS crossbar as ds_bpermute takes).
// Rotating by 8 pairs lane i with lane i ^ 8.  Each step combines a lane's
// value with its partner's by a commutative rule, so afterwards lanes i and
// i ^ 8 hold the same value: the data has period 8, and rotating by 4 then
// reads, in lane i, the value lane i ^ 4 holds; likewise for 2 and 1.  The
// result is therefore bit for bit the xor butterfly's (for NaN-free data,
// where the argmax rule is commutative).
template <int N>
__device__ __forceinline__ int row_ror_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, 0x120 + N, 0xF, 0xF, false);   // DPP row_ror:N
}
template <int N>
__device__ __forceinline__ float row_ror(float v) {
  return __int_as_float(row_ror_i<N>(__float_as_int(v)));
}
// ---- 16-lane group reductions (one MFMA column tile = 16 lanes) ----------
__device__ __forceinline__ float sum16(float v) {
  v += row_ror<8>(v);
  v += row_ror<4>(v);
  v += row_ror<2>(v);
  v += row_ror<1>(v);
  return v;
}
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, row_ror<8>(v));
  v = fmaxf(v, row_ror<4>(v));
  v = fmaxf(v, row_ror<2>(v));
  v = fmaxf(v, row_ror<1>(v));
  return v;
}
template <int N>
__device__ __forceinline__ void argmax_step(float& v, int& idx) {
  const float ov = row_ror<N>(v);
  const int oi = row_ror_i<N>(idx);
  if (ov > v || (ov == v && oi < idx)) { v = ov; idx = oi; }
}
__device__ __forceinline__ void argmax16(float& v, int& idx) {
  argmax_step<8>(v, idx);
  argmax_step<4>(v, idx);
  argmax_step<2>(v, idx);
  argmax_step<1>(v, idx);
}

// ---- wave reductions (butterfly, identical result in every lane) ---------
// Offsets 32 and 16 cross DPP rows (ds_bpermute); 8, 4, 2 and 1 run on row
// rotations in the same order, which gives the same bits (see above).
__device__ __forceinline__ float wave_sum(float v) {
  v += __shfl_xor(v, 32, kWave);
  v += __shfl_xor(v, 16, kWave);
  return sum16(v);
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 32, kWave));
  v = fmaxf(v, __shfl_xor(v, 16, kWave));
  return max16(v);
}
// Max with the lowest index among equal maxima.
__device__ __forceinline__ void wave_argmax(float& v, int& idx) {
#pragma unroll
  for (int o = 32; o > 8; o >>= 1) {
    const float ov = __shfl_xor(v, o, kWave);
    const int oi = __shfl_xor(idx, o, kWave);
    if (ov > v || (ov == v && oi < idx)) { v = ov; idx = oi; }
  }
  argmax16(v, idx);
}
__device__ __forceinline__ int wave_min_int(int v) {
  v = min(v, __shfl_xor(v, 32, kWave));
  v = min(v, __shfl_xor(v, 16, kWave));
  v = min(v, row_ror_i<8>(v));
  v = min(v, row_ror_i<4>(v));
  v = min(v, row_ror_i<2>(v));
  v = min(v, row_ror_i<1>(v));
  return v;
}

// Online-softmax merge of (max, sum of exp((x - max) * invT)) pairs.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2, float invT) {
  if (s2 == 0.0f) return;
  if (s == 0.0f) { m = m2; s = s2; return; }
  if (m2 > m) { s = s * expf((m - m2) * invT) + s2; m = m2; }
  else { s = s + s2 * expf((m2 - m) * invT); }
}
// One butterfly step of wave_lse: partner values m2, s2 from lane i ^ O.
template <int O>
__device__ __forceinline__ void lse_step(float& m, float& s, float m2, float s2, float invT) {
  // merge in a lane-independent order so every lane gets the same bits
  float am = m, as = s, bm = m2, bs = s2;
  const bool swap = (threadIdx.x & O) != 0;
  if (swap) { am = m2; as = s2; bm = m; bs = s; }
  lse_merge(am, as, bm, bs, invT);
  m = am; s = as;
}
__device__ __forceinline__ void wave_lse(float& m, float& s, float invT) {
  lse_step<32>(m, s, __shfl_xor(m, 32, kWave), __shfl_xor(s, 32, kWave), invT);
  lse_step<16>(m, s, __shfl_xor(m, 16, kWave), __shfl_xor(s, 16, kWave), invT);
  lse_step<8>(m, s, row_ror<8>(m), row_ror<8>(s), invT);
  lse_step<4>(m, s, row_ror<4>(m), row_ror<4>(s), invT);
  lse_step<2>(m, s, row_ror<2>(m), row_ror<2>(s), invT);
  lse_step<1>(m, s, row_ror<1>(m), row_ror<1>(s), invT);
}

// Order-preserving map of an fp32 logit to uint32 (larger value, larger key).
__device__ __forceinline__ uint32_t logit_key(float x) {
  const uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}


// Softmax / argmax statistics of one unit of U adjacent 16-column logits
// tiles of a row (U = 1, 2 or 4), one column per lane; the U tiles sit in
// 16-lane groups k U .. k U + U - 1 of the wave, and every lane of the wave
// must call.  Greedy -> (max, lowest argmax); otherwise (max, sum exp((l -
// max)/T)) for p and, for draft rows (i < gamma), the statistics of q' from
// the lane's draft probability qv: T == 1 -> sum q; else (max y, sum exp(y -
// max y)) with y = log(q) / T.  Each tile is reduced over its 16 lanes, then
// the U tiles are merged in a lane-independent order, so every lane holds
// the same bits; the unit's first lane writes when `live`.
__device__ __forceinline__ void lm_unit_stats(float l, bool valid, bool live, int n, int grow,
                                              int unit, int U, int G, int G1, int gamma, int tmode,
                                              float invT, float qv, float* pst, int* pidx,
                                              float* qst) {
  const int lane = threadIdx.x & 63;
  const bool writer = live && (lane & (16 * U - 1)) == 0;
  const size_t t = (size_t)grow * G + unit;
  if (tmode == 0) {
    float v = valid ? l : -INFINITY;
    int idx = valid ? n : 0x7fffffff;
    argmax16(v, idx);
    for (int o = 16; o < 16 * U; o <<= 1) {
      const float ov = __shfl_xor(v, o, kWave);
      const int oi = __shfl_xor(idx, o, kWave);
      if (ov > v || (ov == v && oi < idx)) { v = ov; idx = oi; }
    }
    if (writer) { pst[2 * t] = v; pst[2 * t + 1] = 0.f; pidx[t] = idx; }
    return;
  }
  float mx = max16(valid ? l : -INFINITY);
  float se = sum16(valid ? expf((l - mx) * invT) : 0.f);
  const int b = grow / G1, i = grow - b * G1;
  const bool qrow_ok = live && i < gamma;
  const size_t qrow = (size_t)b * gamma + i;
  if (!(qrow_ok && valid)) qv = 0.f;
  float ym = 0.f, sq;
  if (tmode == 1) {
    sq = sum16(qv);
  } else {
    const float y = qv > 0.f ? logf(qv) * invT : -INFINITY;
    ym = max16(y);
    sq = sum16(qv > 0.f ? expf(y - ym) : 0.f);
  }
  for (int o = 16; o < 16 * U; o <<= 1) {
    const bool swap = (lane & o) != 0;
    float m2 = __shfl_xor(mx, o, kWave), s2 = __shfl_xor(se, o, kWave);
    float am = swap ? m2 : mx, as = swap ? s2 : se, bm = swap ? mx : m2, bs = swap ? se : s2;
    lse_merge(am, as, bm, bs, invT);
    mx = am; se = as;
    const float y2 = __shfl_xor(ym, o, kWave), q2 = __shfl_xor(sq, o, kWave);
    if (tmode == 1) {
      sq = swap ? q2 + sq : sq + q2;
    } else {
      am = swap ? y2 : ym; as = swap ? q2 : sq; bm = swap ? ym : y2; bs = swap ? sq : q2;
      lse_merge(am, as, bm, bs, 1.0f);
      ym = am; sq = as;
    }
  }
  if (writer) { pst[2 * t] = mx; pst[2 * t + 1] = se; }
  if (writer && qrow_ok) {
    const size_t tq = qrow * G + unit;
    qst[2 * tq] = ym;
    qst[2 * tq + 1] = sq;
  }
}

}  // namespace sv
