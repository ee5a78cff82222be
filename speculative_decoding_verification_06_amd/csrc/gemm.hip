// Skinny GEMMs of the target pass, with fused epilogues.
//
// Y[M][N] = X[M][K] @ W[K][N] for M = B * (gamma + 1) rows: the decode
// mat-vec turned into a small mat-mat by scoring every drafted position in
// one pass over the weights ("Speculative decoding" explainer,
// lattice-ai-eng.pages.dev: the single target call over k+1 positions is one
// weight read; "Speculative Decoding: Speeding Sequential Generation",
// aicomputerinstitute.com, Why Generation Is Slow: A Roofline View).  Each
// weight byte is read from HBM once; activations are split once, by the
// kernel that produces them, into bf16 terms for the MFMA path: three exact
// terms in the stacked passes of up to 5 rows, two rounded ones (2^-16
// relative) in the stacked passes of 6 to 8 rows and the wide passes unless
// the exact split is asked for, so the logits track a float64 reference.
//
// Work decomposition: a work group owns NT MFMA column tiles (16 columns
// each) over the whole K range.  Its waves are MG row groups x KG k-groups;
// the k-groups take interleaved 32-row k-steps and are summed through LDS in
// a fixed order, then the same work group runs the epilogue.  No work group
// ever reads another's results: there are no partial buffers, counters or
// device-scope fences (a device-scope release writes back the XCD's L2 and
// costs far more than the weight stream at these sizes), and the sums are
// bit-identical from run to run.

#include <hip/hip_ext.h>

#include "common.h"
#include "internal.h"

#ifndef SV_TARGET_WAVES
#define SV_TARGET_WAVES 2048      // two waves per SIMD over 256 CUs
#endif
#ifndef SV_MIN_BLOCKS
#define SV_MIN_BLOCKS 256         // work groups wanted per GEMM (one per CU)
#endif
#ifndef SV_PIPE_VGPRS
#define SV_PIPE_VGPRS 64          // VGPRs of the load ring per wave
#endif

namespace sv {

// Where a work group has one row group, each weight fragment is loaded by
// one wave, once per pass, so it loads with the non-temporal hint
// (global_load ... nt): the caches stream it instead of holding it over the
// activations, partial sums and draft rows that are read again.  Measured
// on the B = 1 passes, the LM heads went from 48.5 to 43.4 us (32000 x
// 4096) and from 360 to 316 us (128256 x 8192), the up projections from
// 23.7 to 22.2 us.  With two row groups (the 224-row shape) both waves of
// a SIMD load the same fragment and the second relies on the cache: the
// hint there made the greedy pass 4.8% slower, so those loads are plain.
template <bool STREAM>
__device__ __forceinline__ bf16x8 load_weights(const bf16x8* p) {
  if constexpr (STREAM) return __builtin_nontemporal_load(p);
  else return *p;
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

// ---------------------------------------------------------------- epilogues
// res: LDS tile [M][ldr] of finished sums for column tiles c0 .. c0+nt-1.
// Items are (row, 16-column tile) pairs; a wave handles 4 items at a time
// (a round), one per 16-lane group, with one column per lane.
//
// What an epilogue reads from global memory does not depend on the GEMM,
// so epi_prefetch loads it before the k-loop and its latency hides under
// the weight stream instead of adding a round trip to every work group's
// tail.  pv holds, for UP, the first 8 * 64 per-16-column sums of squares
// of the wave's first row; for DOWN and LM, per item of the first
// kPreRounds rounds, the residual h and next gain (DOWN) or the draft
// probability q of the item's column (LM).  Later rounds load on demand.
constexpr int kPreRounds = 4;

struct EpiItem {
  bool live, valid;
  int r, t, tile, n;
  size_t o;
};

__device__ __forceinline__ EpiItem epi_item(const EpiArgs& e, int M, int c0, int nt, int base) {
  const int lane = threadIdx.x & 63;
  EpiItem x;
  const int items = M * nt;
  const int it = base + (lane >> 4);
  x.live = it < items;
  x.r = x.live ? it / nt : 0;
  x.t = x.live ? it - x.r * nt : 0;
  x.tile = c0 + x.t;
  x.n = x.tile * kSub + (lane & 15);
  x.valid = x.live && x.n < e.N;
  x.o = (size_t)x.r * e.ldo + x.n;
  return x;
}

// q value of an LM item (0 for the bonus row, invalid columns or greedy).
__device__ __forceinline__ float lm_item_q(const EpiArgs& e, const EpiItem& x) {
  if (e.tmode == 0 || !x.valid) return 0.f;
  const int grow = e.row0 + x.r;
  const int b = grow / e.G1, i = grow - b * e.G1;
  return i < e.gamma ? e.q[((size_t)b * e.gamma + i) * e.V + x.n] : 0.f;
}

// 1 / rms of row r from its per-16-column sums of squares (one wave; the
// result in every lane): each lane sums a fixed strided subset, then a
// butterfly, in the order run_epilogue uses, so the bits match.
__device__ __forceinline__ float row_inv_rms(const EpiArgs& e, int r) {
  const int lane = threadIdx.x & 63;
  const float* ps = e.ss_in + (size_t)r * e.ss_ld;
  float part[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) part[j] = 0.f;
  for (int t0 = 0; t0 < e.ss_n; t0 += 8 * kWave) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = t0 + j * kWave + lane;
      part[j] += t < e.ss_n ? ps[t] : 0.f;
    }
  }
  float s = ((part[0] + part[1]) + (part[2] + part[3])) + ((part[4] + part[5]) + (part[6] + part[7]));
  s = wave_sum(s);
  return 1.0f / sqrtf(s * e.inv_d + e.eps);
}

__device__ __forceinline__ void epi_prefetch(const EpiArgs& e, int M, int c0, int nt, int nwaves,
                                             float (&pv)[8]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < 8; ++j) pv[j] = 0.f;
  if (e.kind == EPI_UP) {
    if (e.rms) {
      // 1 / rms of rows wave, wave + nwaves, ... (at most 8 per wave)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = wave + j * nwaves;
        pv[j] = r < M ? e.rms[e.row0 + r] : 0.f;
      }
      return;
    }
    if (wave < M) {
      const float* ps = e.ss_in + (size_t)wave * e.ss_ld;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int t = j * kWave + lane;
        pv[j] = t < e.ss_n ? ps[t] : 0.f;
      }
    }
    return;
  }
#pragma unroll
  for (int k = 0; k < kPreRounds; ++k) {
    const EpiItem x = epi_item(e, M, c0, nt, wave * 4 + k * nwaves * 4);
    if (e.kind == EPI_DOWN) {
      pv[2 * k] = x.valid ? e.out[x.o] : 0.f;
      pv[2 * k + 1] = (x.valid && e.gain_next) ? e.gain_next[x.n] : 0.f;
    } else {
      pv[2 * k] = lm_item_q(e, x);
    }
  }
}

// 1 / rms of row `wave` (when < M) from the sums of squares that
// epi_prefetch loaded, into sh_inv.  The MFMA GEMM runs it right after
// issuing its first weight loads, so the butterfly and the square root
// overlap the weight latency instead of lengthening the epilogue; the
// order of the sums is run_epilogue's, so the bits are too.
__device__ __forceinline__ void early_inv_rms(const EpiArgs& e, int M, float* sh_inv,
                                              const float (&pv)[8]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave >= M) return;
  float part[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) part[j] = pv[j];
  const float* ps = e.ss_in + (size_t)wave * e.ss_ld;
  for (int t0 = 8 * kWave; t0 < e.ss_n; t0 += 8 * kWave) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = t0 + j * kWave + lane;
      part[j] += t < e.ss_n ? ps[t] : 0.f;
    }
  }
  float s = ((part[0] + part[1]) + (part[2] + part[3])) + ((part[4] + part[5]) + (part[6] + part[7]));
  s = wave_sum(s);
  if (lane == 0) sh_inv[wave] = 1.0f / sqrtf(s * e.inv_d + e.eps);
}

// rms_early: the UP rows below nwaves already hold 1 / rms in sh_inv
// (early_inv_rms), behind a barrier the caller has passed since.
// XSK: the packing of the split output when the caller knows it at compile
// time (0 plain, 3 stacked three-term, 2 stacked two-term), else -1 and the
// packing comes from e.xs_stack / e.xs_two.
template <int XSK = -1>
__device__ void run_epilogue(const EpiArgs& e, int M, int c0, int nt, const float* res, int ldr,
                             float* sh_inv, int nwaves, const float (&pv)[8],
                             bool rms_early = false) {
  const bool xs_stack = XSK < 0 ? e.xs_stack : XSK != 0;
  const bool xs_two = XSK < 0 ? e.xs_two : XSK == 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15;
  if (e.kind == EPI_UP && e.rms) {
    // prefetched by epi_prefetch for the first 8 rows of each wave
    for (int r = wave, j = 0; r < M; r += nwaves, ++j) {
      float v = 0.f;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        if (jj == j) v = pv[jj];
      if (j >= 8) v = e.rms[e.row0 + r];
      if (lane == 0) sh_inv[r] = v;
    }
    __syncthreads();
  } else if (e.kind == EPI_UP) {
    // 1 / rms per row from its per-16-column sums of squares: one wave per
    // row, each lane summing a fixed strided subset (8 independent loads),
    // then a butterfly; the order is fixed, so the bits are too.  The
    // wave's first row was prefetched; its next three rows are loaded
    // together, so they cost one round trip, not three.
    for (int r0 = wave + (rms_early ? nwaves : 0); r0 < M; r0 += 4 * nwaves) {
      float part[4][8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = r0 + q * nwaves;
        const float* ps = e.ss_in + (size_t)min(r, M - 1) * e.ss_ld;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int t = j * kWave + lane;
          part[q][j] = (q == 0 && r == wave) ? pv[j] : (r < M && t < e.ss_n ? ps[t] : 0.f);
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = r0 + q * nwaves;
        if (r < M) {
          const float* ps = e.ss_in + (size_t)r * e.ss_ld;
          for (int t0 = 8 * kWave; t0 < e.ss_n; t0 += 8 * kWave) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int t = t0 + j * kWave + lane;
              part[q][j] += t < e.ss_n ? ps[t] : 0.f;
            }
          }
          float s = ((part[q][0] + part[q][1]) + (part[q][2] + part[q][3])) +
                    ((part[q][4] + part[q][5]) + (part[q][6] + part[q][7]));
          s = wave_sum(s);
          if (lane == 0) sh_inv[r] = 1.0f / sqrtf(s * e.inv_d + e.eps);
        }
      }
    }
    if (!rms_early || M > nwaves) __syncthreads();
  }
  const int items = M * nt;
  int k = 0;
  for (int base = wave * 4; base < items; base += nwaves * 4, ++k) {
    const EpiItem x = epi_item(e, M, c0, nt, base);
    const bool pre = k < kPreRounds;
    float p0 = 0.f, p1 = 0.f;
#pragma unroll
    for (int kk = 0; kk < kPreRounds; ++kk)
      if (k == kk) { p0 = pv[2 * kk]; p1 = pv[2 * kk + 1]; }
    const float v = x.live ? res[x.r * ldr + x.t * kSub + c] : 0.f;
    // columns past the next GEMM's k-steps have no fragment
    const bool to_xs = e.xs != nullptr && x.live && x.n < kKStep * e.xs_ks;
    if (e.kind == EPI_UP) {
      const float y = x.valid ? silu(v * sh_inv[x.r]) : 0.f;
      if (x.live && !e.xs) e.out[x.o] = y;   // the MFMA path reads only the split copy
      if (to_xs) xs_store(e.xs, x.r, x.n, e.xs_ks, xs_stack, xs_two, y);
    } else if (e.kind == EPI_DOWN) {
      float hn = 0.f;
      if (x.valid) hn = (pre ? p0 : e.out[x.o]) + v;
      if (x.live) e.out[x.o] = hn;
      float y = hn;
      if (e.gain_next) {
        y = x.valid ? hn * (pre ? p1 : e.gain_next[x.n]) : 0.f;
        if (x.live && !e.xs) e.xg[x.o] = y;
        const float sq = sum16(hn * hn);
        if (x.live && c == 0) e.ss_out[(size_t)x.r * e.ss_ld + x.tile] = sq;
      }
      if (to_xs) xs_store(e.xs, x.r, x.n, e.xs_ks, xs_stack, xs_two, y);
    } else {
      if (x.valid && e.out) e.out[x.o] = v;   // no logits buffer: greedy, no debug copy
      const float qv = pre ? p0 : lm_item_q(e, x);
      // one statistics unit per work group and row (its nt tiles)
      lm_unit_stats(v, x.valid, x.live, x.n, e.row0 + x.r, x.tile / nt, nt, e.G, e.G1, e.gamma,
                    e.tmode, e.invT, qv, e.pst, e.pidx, e.qst);
    }
  }
}

// ---------------------------------------------------------------- MFMA GEMM
// bf16 weights in MFMA tiles (layout in internal.h); the activations come
// already split into bf16 terms in A-fragment order (xs_index), so a k-step
// is NT weight fragments + FPT activation fragments per row tile and
// FPT * NT MFMAs, with no vector ALU work.  The stacked packings (SK 3: five
// rows, all three terms in one fragment; SK 2: eight rows, both terms of the
// two-term split in one fragment) cut the activation loads and MFMAs of a
// B = 1 pass by three; the plain packing (16 rows, three fragments) serves
// many rows.  MTW = row tiles per wave,
// MG row groups, NT column tiles per work group; the number of k-groups
// KG = waves / MG is a launch parameter.
// The weight stream is latency bound unless each CU keeps well over 100 KiB
// of loads in flight, so waves run two per SIMD and hold deep register
// pipelines: a k-step stage costs 4 * NT VGPRs of weights and 4 * FPT * MTW
// of activations, and PIPE stages stay within the register budget.
template <int MTW, int NT, bool STACK>
struct MfmaPipe {
  static constexpr int stage = 4 * NT + 4 * (STACK ? 1 : 3) * MTW;
  static constexpr int value = (!STACK && MTW >= 3) ? 2 : (SV_PIPE_VGPRS / stage < 2 ? 2 : SV_PIPE_VGPRS / stage);
};

// SK: the activation packing, 0 plain, 3 stacked with three terms of five
// rows, 2 stacked with two terms of eight rows.
template <int MTW, int MG, int NT, int SK>
__global__ __launch_bounds__(512) void k_gemm_mfma(GemmArgs a) {
  constexpr bool STACK = SK != 0;
  constexpr int PIPE = MfmaPipe<MTW, NT, STACK>::value;
  constexpr int FPT = STACK ? 1 : 3;            // A fragments per row tile and k-step
  constexpr int RPT = SK == 2 ? kStackRows2 : (STACK ? kStackRows : 16);   // rows per row tile
  constexpr int TERMS = STACK ? SK : 1;         // LDS planes per row before the term sum
  extern __shared__ float smem[];
  __shared__ float sh_inv[256];
  const int lane = threadIdx.x & 63;
  const int nwaves = blockDim.x >> 6;
  // wave index as a scalar, so the k-loop branches stay uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int mg = wave % MG, kg = wave / MG, KG = nwaves / MG;
  const int c0 = blockIdx.x * NT;                 // first 16-column tile
  const int M = a.M, KS = a.KS;
  const int mt0 = mg * MTW;
  const int MT = (M + RPT - 1) / RPT;
  // this work group's column block: one contiguous span of KS * NT KiB
  const bf16x8* Wg = reinterpret_cast<const bf16x8*>(a.W) + (size_t)blockIdx.x * KS * NT * 64 + lane;

  f32x4 acc[MTW][NT];
#pragma unroll
  for (int i = 0; i < MTW; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A fragments of each row tile.  Lanes whose A-row holds no real row
  // (past M, or A-row 15 of a stacked tile) read a real row of the same
  // term instead, so every load touches only written memory; their
  // products land in accumulator rows that are never stored.  Tiles past
  // the last read the last one and are not computed.
  const bf16x8* xsrow[MTW];
#pragma unroll
  for (int i = 0; i < MTW; ++i) {
    const int mt = min(mt0 + i, MT - 1);
    const int rows = min(RPT, M - mt * RPT);
    const int ar = lane & 15;
    int al;
    if (STACK) {
      const int p = min(ar / RPT, TERMS - 1);
      al = (lane & 48) + p * RPT + min(ar - p * RPT, rows - 1);
    } else {
      al = (lane & 48) + min(ar, rows - 1);
    }
    xsrow[i] = reinterpret_cast<const bf16x8*>(a.XS) + (size_t)mt * (KS + 1) * FPT * 64 + al;
  }
  const bool wave_live = mt0 < MT;
  float pv[8];
  epi_prefetch(a.e, M, c0, NT, nwaves, pv);

  bf16x8 bq[PIPE][NT];
  bf16x8 xq[PIPE][MTW][FPT];

  // kw: weight k-step; ka: activation k-step (KS = the all-zero step)
#define SV_LOAD(u, kw, ka)                                                       \
  {                                                                              \
    const bf16x8* wp = Wg + (size_t)(kw) * NT * 64;                              \
    _Pragma("unroll") for (int t = 0; t < NT; ++t) bq[u][t] = load_weights<MG == 1>(wp + t * 64);        \
    _Pragma("unroll") for (int i = 0; i < MTW; ++i) {                            \
      const bf16x8* xp = xsrow[i] + (size_t)(ka) * FPT * 64;                     \
      _Pragma("unroll") for (int p = 0; p < FPT; ++p) xq[u][i][p] = xp[p * 64];  \
    }                                                                            \
  }

  // terms outermost: consecutive MFMAs write different accumulators, so none
  // waits on the one before it
#define SV_COMPUTE(u)                                                            \
  {                                                                              \
    _Pragma("unroll") for (int p = 0; p < FPT; ++p) {                            \
      _Pragma("unroll") for (int i = 0; i < MTW; ++i) {                          \
        if (mt0 + i < MT) {                                                      \
          _Pragma("unroll") for (int t = 0; t < NT; ++t)                         \
            acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xq[u][i][p], bq[u][t], \
                                                                acc[i][t], 0, 0, 0); \
        }                                                                        \
      }                                                                          \
    }                                                                            \
  }

  // Software pipeline over a ring of PIPE k-steps: each stage is computed,
  // then refilled with the k-step PIPE positions ahead, so PIPE - 1 k-steps
  // of loads stay in flight while one is consumed.  The loop body has no
  // branches: a refill past the wave's last k-step reloads that step's
  // weights (just fetched, so they come from cache) with the all-zero activation step, so its MFMAs
  // add nothing, every path issues the same loads and each wait covers only
  // the oldest stage.  sched_barrier keeps the issue order of the stages.
  // An UP epilogue that sums squares itself takes each wave's first row's
  // 1 / rms while the first k-steps load (the barrier after the partial
  // tiles orders it before its readers).
  const bool rms_early = a.e.kind == EPI_UP && !a.e.rms;
  int k = kg;
  if (wave_live && k < KS) {
    const int n = (KS - k + KG - 1) / KG;            // k-steps of this wave
    const int klast = k + (n - 1) * KG;
#pragma unroll
    for (int u = 0; u < PIPE; ++u) {
      const int kk = k + u * KG;
      SV_LOAD(u, min(kk, klast), kk <= klast ? kk : KS);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (rms_early) early_inv_rms(a.e, M, sh_inv, pv);
    __builtin_amdgcn_sched_barrier(0);
    for (int it = 0; it < n; it += PIPE) {
#pragma unroll
      for (int u = 0; u < PIPE; ++u) {
        SV_COMPUTE(u);

        const int kk = k + (it + u + PIPE) * KG;
        SV_LOAD(u, min(kk, klast), kk <= klast ? kk : KS);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  } else if (rms_early) {
    early_inv_rms(a.e, M, sh_inv, pv);
  }
#undef SV_LOAD
#undef SV_COMPUTE

  // Partial tiles into LDS red[KG][M][TERMS][ldr] (k-group, row, term),
  // then summed in a fixed order (terms from the last to the first, lo +
  // mid + hi or lo + hi, then k-groups in order) into res[M][ldr].  C layout of 16x16 MFMA: lane holds A-rows
  // 4*(lane/16)+j of column lane%16.
  constexpr int NCOL = NT * kSub;
  constexpr int ldr = NCOL + 1;
  float* red = smem;
  const int crow = 4 * (lane >> 4), ccol = lane & 15;
#pragma unroll
  for (int i = 0; i < MTW; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ar = crow + j;
        int row, p = 0;
        if (STACK) {
          p = ar / RPT;
          row = (mt0 + i) * RPT + (ar - p * RPT);
          if (p >= TERMS) row = M;                // A-row 15 of five-row tiles: no row
        } else {
          row = (mt0 + i) * 16 + ar;
        }
        if (mt0 + i < MT && row < M)
          red[(((size_t)kg * M + row) * TERMS + p) * ldr + t * kSub + ccol] = acc[i][t][j];
      }
  __syncthreads();
  float* res = red;
  if (STACK) {
    res = red + (size_t)KG * M * TERMS * ldr;
    for (int idx = threadIdx.x; idx < M * NCOL; idx += blockDim.x) {
      const int r = idx / NCOL, col = idx - r * NCOL;
      float v = 0.f;
      for (int q = 0; q < KG; ++q) {
        const float* pr = red + (((size_t)q * M + r) * TERMS) * ldr + col;
        v += SK == 2 ? pr[ldr] + pr[0] : (pr[2 * ldr] + pr[ldr]) + pr[0];
      }
      res[r * ldr + col] = v;
    }
    __syncthreads();
  } else if (KG > 1) {
    for (int idx = threadIdx.x; idx < M * NCOL; idx += blockDim.x) {
      const int r = idx / NCOL, col = idx - r * NCOL;
      float v = 0.f;
      for (int q = 0; q < KG; ++q) v += red[((size_t)q * M + r) * ldr + col];
      red[r * ldr + col] = v;
    }
    __syncthreads();
  }
  run_epilogue<SK>(a.e, M, c0, NT, res, ldr, sh_inv, nwaves, pv, rms_early);
}

// ---------------------------------------------------------------- LM epilogue from registers
// In the 16x16 MFMA C layout, register j of the 16-lane group g holds row
// 4 g + j of a tile, one column per lane.  A row's unit statistics reduce
// each lane's columns first and then the 16-lane group, one butterfly per
// statistic: the row max (or argmax), then the sum of exp((l - max) / T).
// They are the separate epilogue's quantities, not its bits (that one
// reduces tile by tile and merges).
// The sums use the hardware exp2 / log2 (__expf, __logf): a relative error
// of about |x| 2^-24 per term, below 2e-6 for every term that is not
// negligible, so 1/Z and the probabilities built on it stay far inside
// their 1e-5 bound; the max is exact.
// The statistics mode TM (0 greedy, 1 T = 1, 2 other T) is a template
// parameter, so the code a wave runs after its k-loop holds one variant
// (deciding the mode per row, fully unrolled, the 72-row LM head kernel was
// 78 KB of code; now 31 KB).
//
// Statistics of one row's unit from its four tiles (one column per lane of
// each tile's 16-lane group); the group's first lane writes when `live`.
template <int TM>
__device__ __forceinline__ void unit_stats_4(const EpiArgs& e, const float (&lv)[4], const float (&qa)[4],
                                             int n0, bool live, int grow, int unit) {
  const bool writer = live && (threadIdx.x & 15) == 0;
  const size_t ts = (size_t)grow * e.G + unit;
  if constexpr (TM == 0) {
    // the lane's four columns first, then one 16-lane butterfly: the
    // largest value with the lowest id is the same in any order
    float v = -INFINITY;
    int idx = 0x7fffffff;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int n = n0 + t * kSub;
      if (live && n < e.N && (lv[t] > v || idx == 0x7fffffff)) { v = lv[t]; idx = n; }
    }
    argmax16(v, idx);
    if (writer) { e.pst[2 * ts] = v; e.pst[2 * ts + 1] = 0.f; e.pidx[ts] = idx; }
    return;
  } else {
    // max over the lane's columns, then over the group; then the sum of
    // exp((l - max) / T) the same way (one butterfly per statistic instead
    // of one per tile and a merge)
    float m = -INFINITY, ymax = -INFINITY;
    float y[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bool valid = live && n0 + t * kSub < e.N;
      if (valid) m = fmaxf(m, lv[t]);
      y[t] = -INFINITY;
      if constexpr (TM == 2) {
        if (valid && qa[t] > 0.f) y[t] = __logf(qa[t]) * e.invT;
        ymax = fmaxf(ymax, y[t]);
      }
    }
    const float mx = max16(m);
    float se = 0.f, sq = 0.f;
    if constexpr (TM == 2) ymax = max16(ymax);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bool valid = live && n0 + t * kSub < e.N;
      if (valid) se += __expf((lv[t] - mx) * e.invT);
      if constexpr (TM == 1) {
        if (valid) sq += qa[t];
      } else {
        if (y[t] > -INFINITY) sq += __expf(y[t] - ymax);
      }
    }
    se = sum16(se);
    sq = sum16(sq);
    if (writer) { e.pst[2 * ts] = mx; e.pst[2 * ts + 1] = se; }
    const int b = grow / e.G1, ip = grow - b * e.G1;
    if (writer && ip < e.gamma) {
      const size_t tq = ((size_t)b * e.gamma + ip) * e.G + unit;
      e.qst[2 * tq] = TM == 1 ? 0.f : ymax;
      e.qst[2 * tq + 1] = sq;
    }
  }
}

// Two-tile variant (NTC = 2: a 64-column unit spans the tiles of waves
// 2u and 2u + 1).  Each wave reduces its two tiles of a row and merges
// them (t0, t1) or (t2, t3); the halves meet in LDS and are merged last,
// the order lm_unit_stats uses.
struct HalfStats { float mx, se, ym, sq; };   // greedy: mx = max logit, se = argmax id bits

template <int TM>
__device__ __forceinline__ HalfStats half_stats_2(const EpiArgs& e, const float (&lv)[2],
                                                  const float (&qa)[2], int n0, bool live) {
  HalfStats h;
  if constexpr (TM == 0) {
    float v = -INFINITY;
    int idx = 0x7fffffff;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int n = n0 + t * kSub;
      if (live && n < e.N && (lv[t] > v || idx == 0x7fffffff)) { v = lv[t]; idx = n; }
    }
    argmax16(v, idx);
    h.mx = v; h.se = __int_as_float(idx); h.ym = 0.f; h.sq = 0.f;
    return h;
  } else {
    float m = -INFINITY, ymax = -INFINITY;
    float y[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bool valid = live && n0 + t * kSub < e.N;
      if (valid) m = fmaxf(m, lv[t]);
      y[t] = -INFINITY;
      if constexpr (TM == 2) {
        if (valid && qa[t] > 0.f) y[t] = __logf(qa[t]) * e.invT;
        ymax = fmaxf(ymax, y[t]);
      }
    }
    const float mx = max16(m);
    float se = 0.f, sq = 0.f;
    if constexpr (TM == 2) ymax = max16(ymax);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bool valid = live && n0 + t * kSub < e.N;
      if (valid) se += __expf((lv[t] - mx) * e.invT);
      if constexpr (TM == 1) {
        if (valid) sq += qa[t];
      } else {
        if (y[t] > -INFINITY) sq += __expf(y[t] - ymax);
      }
    }
    h.mx = mx; h.se = sum16(se); h.ym = TM == 1 ? 0.f : ymax; h.sq = sum16(sq);
    return h;
  }
}

// Draft probabilities of row tile mt's items for NTC column tiles (0 for
// bonus rows, columns past N, greedy passes).
template <int NTC>
__device__ __forceinline__ void wide_lm_q(const EpiArgs& e, float (&qv)[NTC][4], int M, int MT, int mt,
                                          int n0, bool unit_ok) {
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = mt * 16 + 4 * g + j;
    const bool live = unit_ok && mt < MT && row < M;
    const int grow = e.row0 + row;
    const int b = grow / e.G1, ip = grow - b * e.G1;
    const bool qrow = live && e.tmode != 0 && ip < e.gamma;
    const float* qp = e.q + ((size_t)b * e.gamma + (qrow ? ip : 0)) * e.V;
#pragma unroll
    for (int t = 0; t < NTC; ++t) {
      const int n = n0 + t * kSub;
      qv[t][j] = qrow && n < e.N ? qp[n] : 0.f;
    }
  }
}

// Logits and half-unit statistics (to LDS half[row]) of the wave's row
// tiles, two column tiles each (one row group, few accumulators), one tile
// per iteration of a loop that is not unrolled: tile I's accumulators are
// picked out with constant indices, so they stay in registers.
template <int MTW, int NTC, int TM>
__device__ __forceinline__ void wide_lm_tiles(const EpiArgs& e, const f32x4 (&acc)[MTW][NTC], int M, int MT,
                                              int mt0, int unit, int n0, bool unit_ok, float4* half) {
  static_assert(NTC == 2, "two column tiles per wave");
  (void)unit;
  const int g = (threadIdx.x & 63) >> 4;
  // draft probabilities two tiles ahead of the work that uses them (their
  // loads queue behind the other group's weight stream on the CU)
  float qv[NTC][4], qn[NTC][4];
  wide_lm_q<NTC>(e, qv, M, MT, mt0, n0, unit_ok);
  wide_lm_q<NTC>(e, qn, M, MT, MTW > 1 ? mt0 + 1 : MT, n0, unit_ok);
#pragma unroll 1
  for (int I = 0; I < MTW; ++I) {
    f32x4 at[NTC];
#pragma unroll
    for (int t = 0; t < NTC; ++t) at[t] = acc[0][t];
#pragma unroll
    for (int i = 1; i < MTW; ++i)
      if (i == I) {
#pragma unroll
        for (int t = 0; t < NTC; ++t) at[t] = acc[i][t];
      }
    float qnn[NTC][4];
    wide_lm_q<NTC>(e, qnn, M, MT, I + 2 < MTW ? mt0 + I + 2 : MT, n0, unit_ok);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = (mt0 + I) * 16 + 4 * g + j;
      const bool live = unit_ok && mt0 + I < MT && row < M;
      float lv[NTC], qj[NTC];
#pragma unroll
      for (int t = 0; t < NTC; ++t) {
        lv[t] = at[t][j];
        qj[t] = qv[t][j];
        const int n = n0 + t * kSub;
        if (live && n < e.N && e.out) e.out[(size_t)row * e.ldo + n] = lv[t];
      }
      const HalfStats h = half_stats_2<TM>(e, lv, qj, n0, live);
      if ((threadIdx.x & 15) == 0 && mt0 + I < MT) half[row] = make_float4(h.mx, h.se, h.ym, h.sq);
    }
#pragma unroll
    for (int t = 0; t < NTC; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) { qv[t][j] = qn[t][j]; qn[t][j] = qnn[t][j]; }
  }
}

template <int I, int MTW, int TM>
__device__ __forceinline__ void wide_lm_rows4(const EpiArgs& e, const f32x4 (&acc)[MTW][4],
                                              const float (&qv)[4][4], int M, int MT, int mt0,
                                              int unit, int n0, bool unit_ok) {
  float qn[4][4];
  if constexpr (I + 1 < MTW) wide_lm_q<4>(e, qn, M, MT, mt0 + I + 1, n0, unit_ok);
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (mt0 + I) * 16 + 4 * g + j;
    const bool live = unit_ok && mt0 + I < MT && row < M;
    float lv[4], qj[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      lv[t] = acc[I][t][j];
      qj[t] = qv[t][j];
      const int n = n0 + t * kSub;
      if (live && n < e.N && e.out) e.out[(size_t)row * e.ldo + n] = lv[t];
    }
    unit_stats_4<TM>(e, lv, qj, n0, live, e.row0 + row, unit);
  }
  if constexpr (I + 1 < MTW) wide_lm_rows4<I + 1, MTW, TM>(e, acc, qn, M, MT, mt0, unit, n0, unit_ok);
}

template <int MTW, int NTC, int TM>
__device__ __forceinline__ void wide_lm_mode(const EpiArgs& e, const f32x4 (&acc)[MTW][NTC], int M, int MT,
                                             int mt0, int unit, int n0, bool unit_ok, float4* half) {
  if constexpr (NTC == 4) {
    float q0[4][4];
    wide_lm_q<4>(e, q0, M, MT, mt0, n0, unit_ok);
    wide_lm_rows4<0, MTW, TM>(e, acc, q0, M, MT, mt0, unit, n0, unit_ok);
  } else {
    wide_lm_tiles<MTW, NTC, TM>(e, acc, M, MT, mt0, unit, n0, unit_ok, half);
  }
}

template <int MTW, int NTC>
__device__ __forceinline__ void wide_lm_tiles_tm(const EpiArgs& e, const f32x4 (&acc)[MTW][NTC], int M,
                                                 int MT, int mt0, int unit, int n0, bool unit_ok,
                                                 float4* half) {
  if (e.tmode == 0) wide_lm_mode<MTW, NTC, 0>(e, acc, M, MT, mt0, unit, n0, unit_ok, half);
  else if (e.tmode == 1) wide_lm_mode<MTW, NTC, 1>(e, acc, M, MT, mt0, unit, n0, unit_ok, half);
  else wide_lm_mode<MTW, NTC, 2>(e, acc, M, MT, mt0, unit, n0, unit_ok, half);
}

// The LM head's epilogue straight from a wide-GEMM wave's accumulators,
// when one work group sums all of K for its columns.  A wave's four column
// tiles are one 64-column statistics unit.
template <int MTW>
__device__ __forceinline__ void wide_lm_epilogue(const EpiArgs& e, const f32x4 (&acc)[MTW][4], int M,
                                                 int MT, int mt0, int unit, int tiles) {
  const int n0 = unit * 4 * kSub + (threadIdx.x & 15);   // this lane's column in tile 0
  wide_lm_tiles_tm<MTW, 4>(e, acc, M, MT, mt0, unit, n0, unit * 4 < tiles, nullptr);
}

// LM epilogue of the two-tile wide GEMM: CG waves, CG / 2 units per work
// group, rows of all MG row groups; hbuf is LDS for CG * R float4 (R rows).
template <int MTW, int CG>
__device__ __forceinline__ void wide_lm_epilogue2(const EpiArgs& e, const f32x4 (&acc)[MTW][2], int M,
                                                  int MT, int mt0, int cg, int tiles, float4* hbuf,
                                                  int R) {
  const int unit = blockIdx.x * (CG / 2) + cg / 2;
  const int n0 = (unit * 4 + 2 * (cg & 1)) * kSub + (threadIdx.x & 15);
  wide_lm_tiles_tm<MTW, 2>(e, acc, M, MT, mt0, unit, n0, unit * 4 < tiles, hbuf + cg * R);
  __syncthreads();
  for (int k = threadIdx.x; k < (CG / 2) * M; k += blockDim.x) {
    const int u = k / M, row = k - u * M;
    const int ug = blockIdx.x * (CG / 2) + u;
    if (ug * 4 >= tiles) continue;
    float4 lo = hbuf[(2 * u) * R + row];
    const float4 hi = hbuf[(2 * u + 1) * R + row];
    const int grow = e.row0 + row;
    const size_t ts = (size_t)grow * e.G + ug;
    if (e.tmode == 0) {
      const int li = __float_as_int(lo.y), hi_i = __float_as_int(hi.y);
      if (hi.x > lo.x || (hi.x == lo.x && hi_i < li)) { lo.x = hi.x; lo.y = hi.y; }
      e.pst[2 * ts] = lo.x;
      e.pst[2 * ts + 1] = 0.f;
      e.pidx[ts] = __float_as_int(lo.y);
      continue;
    }
    lse_merge(lo.x, lo.y, hi.x, hi.y, e.invT);
    if (e.tmode == 1) lo.w = lo.w + hi.w;
    else lse_merge(lo.z, lo.w, hi.z, hi.w, 1.0f);
    e.pst[2 * ts] = lo.x;
    e.pst[2 * ts + 1] = lo.y;
    const int b = grow / e.G1, ip = grow - b * e.G1;
    if (ip < e.gamma) {
      const size_t tq = ((size_t)b * e.gamma + ip) * e.G + ug;
      e.qst[2 * tq] = lo.z;
      e.qst[2 * tq + 1] = lo.w;
    }
  }
}

// ---------------------------------------------------------------- wide MFMA GEMM
// Many rows (plain packing, 9 to 224 rows): the split activations of a
// k-step, MT row tiles x TERMS terms, are staged once per work group in LDS and
// shared by the group's 16 column tiles (256 columns), instead of being
// read from L2 by every 16-column tile.  MG x CG waves: row groups of MTW
// tiles times column groups of NTC tiles.  A fragments are loaded ahead
// into registers, written to a double-buffered LDS tile, and read back one
// row tile at a time with ds_read_b128; weights stream into a register
// ring.  When the column blocks cannot fill the chip, K is split over
// blockIdx.y and the slices are summed, in slice order, by k_epi_wide8 (UP,
// DOWN) or k_epi_wide (an LM head in slices).
// TERMS: the bf16 terms of each activation read (3, or 2 with the
// two-term split, whose third fragment is skipped).
// Output: fp32 partial sums P[slice][row][col].
template <int MTW, int NTC, int MG, int CG, int RING, int TERMS>
__global__ __launch_bounds__(64 * MG * CG) void k_gemm_wide(WideArgs a, EpiArgs e) {
  // Load vmcnt completes in issue order, so waiting for the activations of
  // the next k-step also waits for every weight load issued before them:
  // a weight ring deeper than the A register sets would gain nothing, so
  // both are RING deep: a k-step's A is loaded RING steps ahead into one
  // of RING register sets.  4 where the registers allow it, 2 where the
  // accumulators take them or two groups must share a CU.
  constexpr int kWideRing = RING;
  constexpr int ASETS = RING;
  // Long k-steps (two row groups): with A loaded two or more steps ahead,
  // the next step's A goes to LDS after the first row tile, so the wait for
  // its writes is not at the barrier, where both waves of a SIMD would idle
  // the MFMA pipe.  (Measured: +2% greedy; the short one-row-group k-steps
  // of 72 rows lose 1%, so they store last.)
  constexpr bool kEarlyStore = ASETS >= 2 && MG == 2;
  static_assert(kWideRing % 2 == 0 && kWideRing % ASETS == 0, "ring slots must map to fixed A sets");
  constexpr int NW = MG * CG, THREADS = 64 * NW;
  static_assert(TERMS == 2 || TERMS == 3, "two or three activation terms");
  constexpr int CPT = (MTW * MG * TERMS * 64 + THREADS - 1) / THREADS;   // A chunks per thread
  extern __shared__ bf16x8 lds_a[];                                   // [2][NFRP]
  const int lane = threadIdx.x & 63, tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int mg = wave / CG, cg = wave - mg * CG;
  const int KS = a.KS, MT = a.MT, M = a.M;
  const int s0 = blockIdx.y * a.ks_slice;
  const int s1 = min(KS, s0 + a.ks_slice);
  const int nsteps = s1 - s0;
  const int nfr = MT * TERMS * 64;
  const bf16x8* XS = reinterpret_cast<const bf16x8*>(a.XS);
  const bf16x8* W = reinterpret_cast<const bf16x8*>(a.W);
  // UP: 1 / rms of every row once per pass, for the epilogue (slice 0's work
  // groups take 16-row blocks in turn), instead of once per epilogue group
  if (e.kind == EPI_UP && e.rms && blockIdx.y == 0) {
    for (int rb = blockIdx.x; rb * 16 < M; rb += gridDim.x)
      for (int r = rb * 16 + wave; r < min(M, rb * 16 + 16); r += NW) {
        const float v = row_inv_rms(e, r);
        if (lane == 0) e.rms[r] = v;
      }
  }

  // weight fragments of this wave's tiles: tile t of layout block b = t / nt
  const bf16x8* wp[NTC];
  bool tval[NTC];
#pragma unroll
  for (int t = 0; t < NTC; ++t) {
    const int tile = blockIdx.x * (NTC * CG) + cg * NTC + t;
    tval[t] = tile < a.tiles;
    const int tt = min(tile, a.tiles - 1);
    const int b = tt / a.nt, tp = tt - b * a.nt;
    wp[t] = W + ((size_t)b * KS * a.nt + tp) * 64 + lane;
  }
  const size_t wstep = (size_t)a.nt * 64;

  f32x4 acc[MTW][NTC];
#pragma unroll
  for (int i = 0; i < MTW; ++i)
#pragma unroll
    for (int t = 0; t < NTC; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 areg[ASETS][CPT];
  bf16x8 bq[kWideRing][NTC];
  // chunk c of a k-step: fragment (mt, p) = (c / (64 TERMS), c / 64 %
  // TERMS), lane c % 64; a row tile's k-step spans three fragments in
  // memory whatever TERMS is.  The LDS tile is padded to CPT * THREADS
  // chunks so the copy has no per-thread branch; chunks past the real ones
  // copy the last real one.
  constexpr int NFRP = CPT * THREADS;
  const bf16x8* asrc[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = min(tid + i * THREADS, nfr - 1);
    const int mt = c / (TERMS * 64), rem = c - mt * (TERMS * 64);
    asrc[i] = XS + (size_t)mt * (KS + 1) * 192 + rem;
  }
  auto load_a = [&](int set, int s) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) areg[set][i] = asrc[i][(size_t)s * 192];
  };
  auto store_a = [&](int set, int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) lds_a[buf * NFRP + tid + i * THREADS] = areg[set][i];
  };
  // k-step k of the slice: weights clamped to its last step, activations
  // from the all-zero step KS past its end, so padded steps add exactly 0
  auto load_b = [&](int slot, int k) {
    const int ss = s0 + min(k, nsteps - 1);
#pragma unroll
    for (int t = 0; t < NTC; ++t) bq[slot][t] = load_weights<MG == 1>(wp[t] + (size_t)ss * wstep);
  };
  auto a_step = [&](int k) { return k < nsteps ? s0 + k : KS; };

  if (nsteps > 0) {
    // The loop body has no branches (the step count is padded to a whole
    // ring), so every s_waitcnt in it counts exactly the loads issued since
    // the one it needs and the weight ring stays kWideRing steps deep.  A
    // branch around a step would let the compiler assume a path on which
    // the refilled slot is the newest load and drain the ring every step.
    const int npad = (nsteps + kWideRing - 1) / kWideRing * kWideRing;
    load_a(0, a_step(0));
#pragma unroll
    for (int u = 0; u < kWideRing; ++u) load_b(u, u);
    store_a(0, 0);
#pragma unroll
    for (int j = 1; j < ASETS; ++j) load_a(j, a_step(j));
    __syncthreads();
    for (int it = 0; it < npad; it += kWideRing) {
#pragma unroll
      for (int u = 0; u < kWideRing; ++u) {
        const int k = it + u;                 // LDS buffer k & 1 = u & 1
        // A for k-step k + ASETS into set k % ASETS (free: it held A(k),
        // stored at the end of the previous step), issued first
        load_a(u % ASETS, a_step(k + ASETS));
        __builtin_amdgcn_sched_barrier(0);
        // A fragments stream from LDS one row tile (three terms) at a
        // time, the next tile's reads issued before this tile's MFMAs.
        // Tiles past MT repeat the last tile (no branch in the MFMA
        // stream); their rows are never stored.
        const bf16x8* abuf = lds_a + (u & 1) * NFRP + lane;
        bf16x8 af[2][TERMS];
#pragma unroll
        for (int p = 0; p < TERMS; ++p) af[0][p] = abuf[(min(mg * MTW, MT - 1) * TERMS + p) * 64];
#pragma unroll
        for (int i = 0; i < MTW; ++i) {
          if (i + 1 < MTW) {
#pragma unroll
            for (int p = 0; p < TERMS; ++p)
              af[(i + 1) & 1][p] = abuf[(min(mg * MTW + i + 1, MT - 1) * TERMS + p) * 64];
          }
          // Two row groups: the two waves of a SIMD (one per row group)
          // share the MFMA pipe; the one inside a tile's MFMA run keeps
          // issue priority until the run ends (measured +0.7% greedy).
          if constexpr (MG == 2) __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int p = 0; p < TERMS; ++p)
#pragma unroll
            for (int t = 0; t < NTC; ++t)
              acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i & 1][p], bq[u][t], acc[i][t], 0, 0, 0);
          if constexpr (MG == 2) __builtin_amdgcn_s_setprio(0);
          if (kEarlyStore && i == 0) {
            // A(k + 1), loaded a step ago, to the other LDS buffer early:
            // its writes have landed long before the barrier
            __builtin_amdgcn_sched_barrier(0);
            store_a((u + 1) % ASETS, (u + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        load_b(u, k + kWideRing);
        if (!kEarlyStore) {
          // A(k + 1) to the other LDS buffer, last, so its wait comes late
          __builtin_amdgcn_sched_barrier(0);
          store_a((u + 1) % ASETS, (u + 1) & 1);
        }
        __syncthreads();
      }
    }
  }

  if (a.fuse_lm) {
    static_assert(NTC == 4 || (NTC == 2 && CG % 2 == 0), "units of four tiles per wave or wave pair");
    if constexpr (NTC == 4) {
      wide_lm_epilogue<MTW>(e, acc, M, MT, mg * MTW, blockIdx.x * CG + cg, a.tiles);
    } else {
      // the A buffers hold the half-unit statistics (free after the k-loop)
      constexpr int R = MG * MTW * 16;
      static_assert(CG * R * 16 <= 2 * NFRP * 16, "LDS for the half-unit statistics");
      wide_lm_epilogue2<MTW, CG>(e, acc, M, MT, mg * MTW, cg, a.tiles,
                                 reinterpret_cast<float4*>(lds_a), R);
    }
    return;
  }

  // partial sums to P[slice][row][col]; C layout: lane holds rows
  // 4 (lane / 16) + j of column lane % 16
  float* P = a.P + (size_t)blockIdx.y * a.slice_stride;
#pragma unroll
  for (int i = 0; i < MTW; ++i)
#pragma unroll
    for (int t = 0; t < NTC; ++t) {
      const int tile = blockIdx.x * (NTC * CG) + cg * NTC + t;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = (mg * MTW + i) * 16 + 4 * (lane >> 4) + j;
        if (tval[t] && row < M) P[(size_t)row * a.ldp + tile * kSub + (lane & 15)] = acc[i][t][j];
      }
    }
}

// Epilogue arguments of the rows from m0 on (m0 a multiple of 16).
__device__ __forceinline__ EpiArgs epi_rows(const EpiArgs& e, int m0) {
  EpiArgs r = e;
  r.out = e.out ? e.out + (size_t)m0 * e.ldo : nullptr;
  if (e.kind == EPI_UP) r.ss_in = e.ss_in + (size_t)m0 * e.ss_ld;
  if (e.kind == EPI_DOWN) {
    r.xg = e.xg + (size_t)m0 * e.ldo;
    r.ss_out = e.ss_out + (size_t)m0 * e.ss_ld;
  }
  if (e.xs) r.xs = e.xs + (size_t)(m0 / 16) * (e.xs_ks + 1) * 3 * 512;
  r.row0 = e.row0 + m0;
  return r;
}

// Work group (64-column block, 16-row tile): sums the S slices of P (in
// slice order) into an LDS tile and runs the GEMM's epilogue on it.
constexpr int kEpiThreads = 256;
__global__ __launch_bounds__(kEpiThreads) void k_epi_wide(WideArgs a, EpiArgs e0) {
  constexpr int ldr = 4 * kSub + 1;
  __shared__ float res[16 * ldr];
  __shared__ float sh_inv[16];
  const int c0 = blockIdx.x * 4, m0 = blockIdx.y * 16;
  const int M = min(16, a.M - m0);
  const EpiArgs e = epi_rows(e0, m0);
  float pv[8];
  epi_prefetch(e, M, c0, 4, kEpiThreads / kWave, pv);
  // 4 items per thread, all slice loads of a batch of slices in flight
  const int idx0 = threadIdx.x;
  float v[4];
  const float* p[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int idx = min(idx0 + j * kEpiThreads, M * 64 - 1);
    p[j] = a.P + (size_t)(m0 + (idx >> 6)) * a.ldp + c0 * kSub + (idx & 63);
    v[j] = 0.f;
  }
  for (int sl = 0; sl < a.S; sl += 4) {
    float x[4][4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        x[q][j] = sl + q < a.S ? p[j][(size_t)(sl + q) * a.slice_stride] : 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] += x[q][j];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int idx = idx0 + j * kEpiThreads;
    if (idx < M * 64) res[(idx >> 6) * ldr + (idx & 63)] = v[j];
  }
  __syncthreads();
  run_epilogue(e, M, c0, 4, res, ldr, sh_inv, kEpiThreads / kWave, pv);
}

// The UP and DOWN epilogues after K slices with each thread owning 8
// consecutive columns of one row: the slices' partial sums as 16-byte loads
// (summed in slice order), and the split activations for the next GEMM as
// one 16-byte store per term.  Work group: 16 rows x 128 columns.  The same
// arithmetic as run_epilogue's, except that a 16-column subtile's sum of
// squares adds its two halves of 8 (a different rounding order).
constexpr int kEpi8Cols = 128;
__global__ __launch_bounds__(kEpiThreads) void k_epi_wide8(WideArgs a, EpiArgs e0) {
  const int tid = threadIdx.x, r = tid >> 4, cgp = tid & 15;
  const int m0 = blockIdx.y * 16;
  const int n0 = blockIdx.x * kEpi8Cols + 8 * cgp;
  const int M = min(16, a.M - m0);
  const bool live = r < M && n0 < a.ldp;
  const EpiArgs e = epi_rows(e0, m0);
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = 0.f;
  if (live) {
    const float* p = a.P + (size_t)(m0 + r) * a.ldp + n0;
    for (int sl = 0; sl < a.S; sl += 4) {
      float4 x[4][2];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool in = sl + q < a.S;
        const float4* pq = reinterpret_cast<const float4*>(p + (size_t)(in ? sl + q : 0) * a.slice_stride);
        x[q][0] = in ? pq[0] : make_float4(0.f, 0.f, 0.f, 0.f);
        x[q][1] = in ? pq[1] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[0] += x[q][0].x; v[1] += x[q][0].y; v[2] += x[q][0].z; v[3] += x[q][0].w;
        v[4] += x[q][1].x; v[5] += x[q][1].y; v[6] += x[q][1].z; v[7] += x[q][1].w;
      }
    }
  }
  float y[8];
  if (e.kind == EPI_UP) {
    const float inv = live ? e.rms[e.row0 + r] : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = live && n0 + j < e.N ? silu(v[j] * inv) : 0.f;
    if (live && !e.xs)
#pragma unroll
      for (int j = 0; j < 8; ++j) e.out[(size_t)r * e.ldo + n0 + j] = y[j];
  } else {
    float hn[8];
    float* hrow = e.out + (size_t)r * e.ldo + n0;
#pragma unroll
    for (int j = 0; j < 8; ++j) hn[j] = live && n0 + j < e.N ? hrow[j] + v[j] : 0.f;
    if (live)
#pragma unroll
      for (int j = 0; j < 8; ++j) hrow[j] = hn[j];
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = hn[j];
    if (e.gain_next) {
#pragma unroll
      for (int j = 0; j < 8; ++j) y[j] = live && n0 + j < e.N ? hn[j] * e.gain_next[n0 + j] : 0.f;
      if (live && !e.xs)
#pragma unroll
        for (int j = 0; j < 8; ++j) e.xg[(size_t)r * e.ldo + n0 + j] = y[j];
      float sq = ((hn[0] * hn[0] + hn[1] * hn[1]) + (hn[2] * hn[2] + hn[3] * hn[3])) +
                 ((hn[4] * hn[4] + hn[5] * hn[5]) + (hn[6] * hn[6] + hn[7] * hn[7]));
      sq += __shfl_xor(sq, 1, kWave);                 // the subtile's other 8 columns
      if (live && (cgp & 1) == 0) e.ss_out[(size_t)r * e.ss_ld + n0 / kSub] = sq;
    }
  }
  if (live && e.xs && n0 < kKStep * e.xs_ks) {
    uint32_t t[3][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t a0, b0, c0 = 0, a1, b1, c1 = 0;
      if (e.xs_two) { split2_bf16(y[2 * j], a0, b0); split2_bf16(y[2 * j + 1], a1, b1); }
      else { split3_bf16(y[2 * j], a0, b0, c0); split3_bf16(y[2 * j + 1], a1, b1, c1); }
      t[0][j] = a0 | (a1 << 16);
      t[1][j] = b0 | (b1 << 16);
      t[2][j] = c0 | (c1 << 16);
    }
    uint16_t* base = e.xs + xs_index(r, n0, e.xs_ks, false, e.xs_two);
    const int st = xs_term_step(false, e.xs_two);
#pragma unroll
    for (int q = 0; q < 3; ++q)
      if (q < 2 || !e.xs_two) *reinterpret_cast<uint4*>(base + q * st) = make_uint4(t[q][0], t[q][1], t[q][2], t[q][3]);
  }
}

// ---------------------------------------------------------------- vector-FMA GEMM
// Row-major weights (fp32 or bf16), kFmaWaves waves, 4 column tiles (64
// columns) per work group.  Lane = (row r = lane / 8 of an 8-row step, 8
// columns at 8 * (lane % 8)); the waves take interleaved 8-row steps of K,
// kFmaUnroll steps' loads issued together; rows of X are processed 8 at a
// time.  The waves' sums meet in LDS in wave order.
template <typename WT>
__device__ __forceinline__ void load_w8(const WT* p, float (&w)[8]);
template <>
__device__ __forceinline__ void load_w8<float>(const float* p, float (&w)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
  w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}
template <>
__device__ __forceinline__ void load_w8<uint16_t>(const uint16_t* p, float (&w)[8]) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  w[0] = bf16_lo(a.x); w[1] = bf16_hi(a.x); w[2] = bf16_lo(a.y); w[3] = bf16_hi(a.y);
  w[4] = bf16_lo(a.z); w[5] = bf16_hi(a.z); w[6] = bf16_lo(a.w); w[7] = bf16_hi(a.w);
}

constexpr int kFmaThreads = kFmaWaves * kWave;
constexpr int kFmaUnroll = 4;

template <typename WT>
__global__ __launch_bounds__(kFmaThreads) void k_gemm_fma(GemmArgs a) {
  extern __shared__ float smem[];
  __shared__ float sh_inv[256];
  constexpr int ldr = kGroupCols + 1;
  constexpr int kStep = kFmaWaves * 8;             // k rows of one step of the group
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = blockIdx.x;                        // 64-column block
  const int Kp = a.KS * kKStep;
  const int M = a.M;
  const int rr = lane >> 3, cg = (lane & 7) * 8;
  const WT* W = reinterpret_cast<const WT*>(a.W) + (size_t)g * kGroupCols + cg;
  float* res = smem;                       // [M][ldr]
  float* red = smem + M * ldr;             // [kFmaWaves][8][ldr]
  float pv[8];
  epi_prefetch(a.e, M, g * 4, 4, kFmaWaves, pv);

  for (int m0 = 0; m0 < M; m0 += 8) {
    const int mr = min(8, M - m0);
    float acc[8][8];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[m][j] = 0.f;
    for (int k0 = wave * 8 + rr; k0 < Kp; k0 += kStep * kFmaUnroll) {
      // kFmaUnroll steps: every load first (rows past Kp read row Kp - 1
      // and count zero), then the FMAs
      float w[kFmaUnroll][8], xv[kFmaUnroll][8];
#pragma unroll
      for (int u = 0; u < kFmaUnroll; ++u) {
        const int k = k0 + u * kStep;
        load_w8<WT>(W + (size_t)min(k, Kp - 1) * a.Np, w[u]);
#pragma unroll
        for (int m = 0; m < 8; ++m)
          xv[u][m] = m < mr && k < Kp ? a.X[(size_t)(m0 + m) * a.ldx + k] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kFmaUnroll; ++u)
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[m][j] = fmaf(xv[u][m], w[u][j], acc[m][j]);
    }
    // sum the 8 row-lanes that share a column group (lanes differ in bits 3..5)
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float v = acc[m][j];
        v += row_ror<8>(v);                 // lane i ^ 8 of the 16-lane row
        v += __shfl_xor(v, 16, kWave);
        v += __shfl_xor(v, 32, kWave);
        acc[m][j] = v;
      }
    if (rr == 0) {
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int j = 0; j < 8; ++j) red[(wave * 8 + m) * ldr + cg + j] = acc[m][j];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < mr * kGroupCols; idx += kFmaThreads) {
      const int m = idx / kGroupCols, c = idx - m * kGroupCols;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kFmaWaves; ++w) v += red[(w * 8 + m) * ldr + c];
      res[(m0 + m) * ldr + c] = v;
    }
    __syncthreads();
  }
  run_epilogue(a.e, M, g * 4, 4, res, ldr, sh_inv, kFmaWaves, pv);
}

// ---------------------------------------------------------------- host side

int mfma_block_tiles(int Np) {
  // the widest column block (up to 4 tiles) that still gives 7/8 of the CUs
  // a block: 896 tiles take 224 blocks of 4 (one per CU, 8 waves each)
  // rather than 448 of 2 (measured 25.7 -> 24.6 us per 117 MB launch)
  const int tiles = Np / kSub;
  int nt = 4;
  while (nt > 1 && tiles / nt < SV_MIN_BLOCKS * 7 / 8) nt /= 2;
  return nt;
}

GemmPlan plan_gemm(int path, int M, const Mat& m, bool stack, bool two) {
  GemmPlan p;
  p.path = path;
  const int tiles = m.Np / kSub;
  const int KS = m.Kp / kKStep;
  if (path != PATH_MFMA) {
    p.nt = 4; p.mg = 1; p.mtw = 1; p.kg = 4;
    p.blocks = m.Np / kGroupCols;
    p.lds = ((size_t)M * (kGroupCols + 1) + kFmaWaves * 8 * (kGroupCols + 1)) * sizeof(float);
    return p;
  }
  p.stack = stack;
  p.two = stack && two;
  if (p.stack) {
    const int R = xs_stack_rows(p.two);
    p.mtw = (M + R - 1) / R;
    p.mg = 1;
  } else {
    const int MT = (M + 15) / 16;
    if (MT <= 2) { p.mtw = MT; p.mg = 1; }
    else if (MT <= 4) { p.mtw = 2; p.mg = 2; }
    else if (MT <= 6) { p.mtw = 3; p.mg = 2; }
    else if (MT <= 8) { p.mtw = 4; p.mg = 2; }
    else if (MT <= 12) { p.mtw = 3; p.mg = 4; }
    else { p.mtw = 4; p.mg = 4; }
  }
  p.nt = m.nt;
  p.blocks = tiles / p.nt;
  // k-groups: about SV_TARGET_WAVES waves in all, within the work-group
  // size, the k-steps and 64 KiB of LDS for the k-group tiles (plus the
  // summed tile of the stacked packing)
  const int max_waves = 8;
  const size_t ldr = (size_t)p.nt * kSub + 1;
  auto lds_of = [&](int kg) {
    return p.stack ? ((size_t)kg * M * 3 + M) * ldr * sizeof(float)
                   : (size_t)kg * M * ldr * sizeof(float);
  };
  p.kg = 1;
  while (p.mg * p.kg * 2 <= max_waves && (size_t)p.blocks * p.mg * p.kg * 2 <= SV_TARGET_WAVES &&
         p.kg * 2 <= KS && lds_of(p.kg * 2) <= 65536)
    p.kg *= 2;
  p.lds = lds_of(p.kg);
  return p;
}

WidePlan plan_wide(int M, const Mat& m, bool two_term) {
  WidePlan p;
  p.MT = (M + 15) / 16;
  p.terms = two_term ? 2 : 3;
  // two row groups x 4 column groups of 4 tiles = 16 column tiles, 8 waves
  p.mtw = (p.MT + 1) / 2;
  p.mg = 2; p.ntc = 4; p.cg = 4;
  const int tiles = m.Np / kSub;
  // Up to 80 rows, and with two terms up to 160 rows where the 16-tile
  // blocks do not outnumber the CUs: one row group of MT tiles (no padding
  // tile), 8 column groups of 2 tiles, so no two waves load the same weight
  // tile (measured against two row groups with two terms: 88 and 96 rows
  // 9-11% faster per pass, 120 and 128 rows 3-5%, 160 rows 2%, 192 rows
  // 1% slower and 224 rows 6% slower).  When more 16-tile blocks than CUs
  // would run two per CU (the LM head), up to 80 rows, 16 column groups of
  // 1024 threads instead: one group per CU whose waves keep step at the
  // k-step barrier.  Two groups on a CU do not: the older one is served
  // first and finishes its k-loop in about half the time, and the younger
  // one then streams alone, latency bound.
  if (p.MT <= 5 || (two_term && p.MT <= 10 && tiles / 16 <= SV_MIN_BLOCKS)) {
    p.mtw = p.MT; p.mg = 1; p.ntc = 2;
    p.cg = (p.MT <= 5 && tiles / 16 > SV_MIN_BLOCKS) ? 16 : 8;
  } else if (two_term && p.MT >= 11) {
    // 161 to 224 rows with two terms: two row groups of 16 waves, 8 column
    // groups of 2 tiles (123 VGPRs, four waves per SIMD), so a SIMD holds
    // four waves to alternate on the MFMA pipe; each k-step's activations
    // are read from LDS twice as often as with 4 column groups of 4 tiles
    // (measured: greedy pass 4032 -> 3940 and 4094 -> 4017 us in two
    // calls, B = 1 passes of 176 to 224 rows 0.5-3% faster)
    p.ntc = 2; p.cg = 8;
  }
  const int ntw = p.ntc * p.cg;
  p.colblocks = (tiles + ntw - 1) / ntw;
  const int KS = m.Kp / kKStep;
  // K slices: one 8-wave work group fits a CU at a time, so the launch
  // runs in rounds of SV_MIN_BLOCKS groups, and every slice adds an M x N
  // fp32 partial sum written and read back.  Each slice is at least 8
  // k-steps and divides K evenly.  Up to 112 rows the weight stream bounds
  // the launch: take the fewest slices whose rounds are at least 85% full,
  // else the fullest.  Past 112 rows the MFMA work bounds it and every CU
  // runs at its own rate: minimise a cost in k-steps, rounds x (slice
  // length + 2 for a group's start and its partial-sum stores) plus N/6000
  // per slice for the partial's round trip through HBM (a k-step and the
  // partial both scale with M, so M drops out).  Measured at 224 rows, two
  // slices of 128 k-steps in 224 groups beat four of 64 in 448 groups by
  // 3% of the pass, and sixteen slices lose 10%.
  const bool mfma_bound = M > 112;
  int S = 1;
  double best = 0.0, best_cost = -1.0;
  for (int s = 1; s <= 16 && KS / s >= 8; ++s) {
    if (KS % s != 0 && s > 1) continue;
    const int w = p.colblocks * s;
    const int rounds = (w + SV_MIN_BLOCKS - 1) / SV_MIN_BLOCKS;
    if (mfma_bound) {
      const double cost = rounds * (double)((KS + s - 1) / s + 2) + s * (double)m.Np / 6000.0;
      if (best_cost < 0.0 || cost < best_cost - 1e-9) { best_cost = cost; S = s; }
      continue;
    }
    const double eff = (double)w / ((double)rounds * SV_MIN_BLOCKS);
    if (eff > best + 1e-9) { best = eff; S = s; }
    if (eff >= 0.85) { S = s; break; }
  }
  p.ks_slice = (KS + S - 1) / S;
  p.S = (KS + p.ks_slice - 1) / p.ks_slice;
  const int threads = 64 * p.mg * p.cg;
  const int cpt = (p.mtw * p.mg * p.terms * 64 + threads - 1) / threads;
  p.lds = (size_t)2 * cpt * threads * 16;
  return p;
}

template <int MTW, int NTC, int MG, int CG, int RING, int TERMS>
static void launch_wide_t(const WidePlan& p, const WideArgs& a, const EpiArgs& e, hipStream_t st,
                          hipEvent_t e0, hipEvent_t e1) {
  // the double-buffered activation tile can exceed the default 64 KiB
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&k_gemm_wide<MTW, NTC, MG, CG, RING, TERMS>),
      hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
  (void)attr;
  hipExtLaunchKernelGGL((k_gemm_wide<MTW, NTC, MG, CG, RING, TERMS>), dim3(p.colblocks, p.S),
                        dim3(64 * MG * CG), p.lds, st, e0, e1, 0, a, e);
}

template <int TERMS>
static void launch_wide_terms(const WidePlan& p, const WideArgs& a, const EpiArgs& e, hipStream_t st,
                              hipEvent_t e0, hipEvent_t e1) {
  if (p.mg == 1 && p.cg == 16) {
    switch (p.mtw) {
      case 1: launch_wide_t<1, 2, 1, 16, 4, TERMS>(p, a, e, st, e0, e1); break;
      case 2: launch_wide_t<2, 2, 1, 16, 4, TERMS>(p, a, e, st, e0, e1); break;
      case 3: launch_wide_t<3, 2, 1, 16, 4, TERMS>(p, a, e, st, e0, e1); break;
      case 4: launch_wide_t<4, 2, 1, 16, 4, TERMS>(p, a, e, st, e0, e1); break;
      // four waves per SIMD: 128 VGPRs hold a 4-deep ring with two terms
      default: launch_wide_t<5, 2, 1, 16, TERMS == 2 ? 4 : 2, TERMS>(p, a, e, st, e0, e1); break;
    }
  } else if (p.mg == 1) {
    switch (p.mtw) {
      case 1: launch_wide_t<1, 2, 1, 8, 4, TERMS>(p, a, e, st, e0, e1); break;
      case 2: launch_wide_t<2, 2, 1, 8, 4, TERMS>(p, a, e, st, e0, e1); break;
      case 3: launch_wide_t<3, 2, 1, 8, 4, TERMS>(p, a, e, st, e0, e1); break;
      case 4: launch_wide_t<4, 2, 1, 8, 4, TERMS>(p, a, e, st, e0, e1); break;
      // 6 to 10 row tiles (two terms): a 2-deep ring, 123-160 VGPRs
      case 6: launch_wide_t<6, 2, 1, 8, 2, TERMS>(p, a, e, st, e0, e1); break;
      case 7: launch_wide_t<7, 2, 1, 8, 2, TERMS>(p, a, e, st, e0, e1); break;
      case 8: launch_wide_t<8, 2, 1, 8, 2, TERMS>(p, a, e, st, e0, e1); break;
      case 9: launch_wide_t<9, 2, 1, 8, 2, TERMS>(p, a, e, st, e0, e1); break;
      case 10: launch_wide_t<10, 2, 1, 8, 2, TERMS>(p, a, e, st, e0, e1); break;
      default:
        // a 4-deep ring takes 137 registers with three terms: one group per
        // CU.  Where more groups than CUs are launched, two groups per CU
        // with a 2-deep ring stream faster (measured on a 501-group LM
        // head, now launched in the 1024-thread shape above).
        if (p.colblocks * p.S > SV_MIN_BLOCKS) launch_wide_t<5, 2, 1, 8, 2, TERMS>(p, a, e, st, e0, e1);
        else launch_wide_t<5, 2, 1, 8, 4, TERMS>(p, a, e, st, e0, e1);
        break;
    }
  } else if (p.ntc == 2) {
    if constexpr (TERMS == 2) {   // 11 to 14 row tiles in two row groups of 8 column groups
      if (p.mtw == 6) launch_wide_t<6, 2, 2, 8, 2, TERMS>(p, a, e, st, e0, e1);
      else launch_wide_t<7, 2, 2, 8, 2, TERMS>(p, a, e, st, e0, e1);
    }
  } else {
    switch (p.mtw) {   // 6 to 14 row tiles in two row groups: mtw = 3 .. 7
      case 3: launch_wide_t<3, 4, 2, 4, 4, TERMS>(p, a, e, st, e0, e1); break;
      case 4: launch_wide_t<4, 4, 2, 4, 4, TERMS>(p, a, e, st, e0, e1); break;
      case 5: launch_wide_t<5, 4, 2, 4, 2, TERMS>(p, a, e, st, e0, e1); break;
      case 6: launch_wide_t<6, 4, 2, 4, 2, TERMS>(p, a, e, st, e0, e1); break;
      default: launch_wide_t<7, 4, 2, 4, 2, TERMS>(p, a, e, st, e0, e1); break;
    }
  }
}

hipError_t launch_wide(const WidePlan& p, const WideArgs& a_in, const EpiArgs& e, hipStream_t st,
                       hipEvent_t e0, hipEvent_t e1) {
  WideArgs a = a_in;
  a.fuse_lm = p.S == 1 && e.kind == EPI_LM;
  // plan_wide gives two row groups of 2-tile column groups only with two
  // terms; no other plan reaches that shape's launch
  if (p.mg == 2 && p.ntc == 2 && p.terms != 2) return hipErrorInvalidValue;
  if (p.terms == 2) launch_wide_terms<2>(p, a, e, st, e0, e1);
  else launch_wide_terms<3>(p, a, e, st, e0, e1);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.fuse_lm) return err;
  if (e.kind == EPI_LM)
    hipLaunchKernelGGL(k_epi_wide, dim3(a.tiles / 4, (a.M + 15) / 16), dim3(kEpiThreads), 0, st, a, e);
  else
    hipLaunchKernelGGL(k_epi_wide8, dim3((a.ldp + kEpi8Cols - 1) / kEpi8Cols, (a.M + 15) / 16),
                       dim3(kEpiThreads), 0, st, a, e);
  return hipGetLastError();
}

// Launches go through hipExtLaunchKernelGGL so that, when timing is on, the
// two events take the kernel's own start and end timestamps (no extra
// packets between kernels).
template <int MTW, int MG, int SK>
static hipError_t launch_mfma_mg(const GemmPlan& p, const GemmArgs& a, hipStream_t st,
                                 hipEvent_t e0, hipEvent_t e1) {
  const dim3 grid(p.blocks), block(64 * p.mg * p.kg);
  switch (p.nt) {
    case 1: hipExtLaunchKernelGGL((k_gemm_mfma<MTW, MG, 1, SK>), grid, block, p.lds, st, e0, e1, 0, a); break;
    case 2: hipExtLaunchKernelGGL((k_gemm_mfma<MTW, MG, 2, SK>), grid, block, p.lds, st, e0, e1, 0, a); break;
    default: hipExtLaunchKernelGGL((k_gemm_mfma<MTW, MG, 4, SK>), grid, block, p.lds, st, e0, e1, 0, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmPlan& p, const GemmArgs& a, hipStream_t st, hipEvent_t e0,
                       hipEvent_t e1) {
  if (p.path == PATH_FMA_F32 || p.path == PATH_FMA_BF16) {
    const dim3 grid(p.blocks), block(kFmaThreads);
    if (p.path == PATH_FMA_F32)
      hipExtLaunchKernelGGL((k_gemm_fma<float>), grid, block, p.lds, st, e0, e1, 0, a);
    else
      hipExtLaunchKernelGGL((k_gemm_fma<uint16_t>), grid, block, p.lds, st, e0, e1, 0, a);
    return hipGetLastError();
  }
  if (p.stack && p.two) return launch_mfma_mg<1, 1, 2>(p, a, st, e0, e1);   // 6 to 8 rows
  if (p.stack)
    return p.mtw == 1 ? launch_mfma_mg<1, 1, 3>(p, a, st, e0, e1)
                      : launch_mfma_mg<2, 1, 3>(p, a, st, e0, e1);
  if (p.mg == 1)
    return p.mtw == 1 ? launch_mfma_mg<1, 1, 0>(p, a, st, e0, e1)
                      : launch_mfma_mg<2, 1, 0>(p, a, st, e0, e1);
  if (p.mg == 2) {
    if (p.mtw == 2) return launch_mfma_mg<2, 2, 0>(p, a, st, e0, e1);
    if (p.mtw == 3) return launch_mfma_mg<3, 2, 0>(p, a, st, e0, e1);
    return launch_mfma_mg<4, 2, 0>(p, a, st, e0, e1);
  }
  return p.mtw == 3 ? launch_mfma_mg<3, 4, 0>(p, a, st, e0, e1)
                    : launch_mfma_mg<4, 4, 0>(p, a, st, e0, e1);
}

}  // namespace sv
