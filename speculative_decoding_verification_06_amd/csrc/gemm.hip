// Split-K skinny GEMMs of the target pass, with fused epilogues.
//
// Y[M][N] = X[M][K] @ W[K][N] for M = B * (gamma + 1) rows: the decode
// mat-vec turned into a small mat-mat by scoring every drafted position in
// one pass over the weights ("Speculative decoding" explainer,
// lattice-ai-eng.pages.dev: the single target call over k+1 positions is one
// weight read; "Speculative Decoding: Speeding Sequential Generation",
// aicomputerinstitute.com, Why Generation Is Slow: A Roofline View).  Each
// weight byte is read from HBM once; activations stay fp32 (MFMA path:
// split into bf16 hi/mid/lo terms) so the logits track a float64 reference.
//
// Work decomposition: work group = 4 waves on one column group of 64
// columns and one k-range (split) of the weights.  When a column group has
// S > 1 splits, every work group writes its partial tile, and the last one
// to arrive (device-scope counter) sums the S partials in split order and
// runs the epilogue, so results do not depend on arrival order.

#include "common.h"
#include "internal.h"

namespace sv {

constexpr int kThreads = 256;
constexpr int kResLd = kGroupCols + 1;   // padded LDS row of the result tile

__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

// ---------------------------------------------------------------- epilogues
// res: LDS tile [M][kResLd] holding the finished sums for this column group.
template <int EPI>
__device__ void run_epilogue(const EpiArgs& e, int M, int g, const float* res, float* sh_rowv) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = g * kGroupCols + lane;
  const bool valid = n < e.N;
  if constexpr (EPI == EPI_UP) {
    for (int r = threadIdx.x; r < M; r += kThreads) {
      float s = 0.f;
      for (int t = 0; t < e.ss_n; ++t) s += e.ss_in[(size_t)r * e.ss_ld + t];
      sh_rowv[r] = 1.0f / sqrtf(s * e.inv_d + e.eps);
    }
    __syncthreads();
    for (int r = wave; r < M; r += 4) {
      const float v = res[r * kResLd + lane];
      e.out[(size_t)r * e.ldo + n] = valid ? silu(v * sh_rowv[r]) : 0.f;
    }
  } else if constexpr (EPI == EPI_DOWN) {
    for (int r = wave; r < M; r += 4) {
      float hn = 0.f;
      if (valid) hn = e.out[(size_t)r * e.ldo + n] + res[r * kResLd + lane];
      e.out[(size_t)r * e.ldo + n] = hn;
      if (e.gain_next) {
        e.xg[(size_t)r * e.ldo + n] = valid ? hn * e.gain_next[n] : 0.f;
        const float sq = wave_sum(hn * hn);
        if (lane == 0) e.ss_out[(size_t)r * e.ss_ld + g] = sq;
      }
    }
  } else {  // EPI_LM
    for (int r = wave; r < M; r += 4) {
      const float l = res[r * kResLd + lane];
      if (valid) e.out[(size_t)r * e.ldo + n] = l;
      lm_tile_stats(l, valid, n, e.row0 + r, g, e.G, e.G1, e.gamma, e.V, e.tmode, e.invT,
                    e.q, e.pst, e.pidx, e.qst);
    }
  }
}

// Publish this work group's tile; return true in the work group that must
// finish the column group (then res holds the split-ordered total).
__device__ bool splitk_finish(const GemmArgs& a, int g, int s, float* res, int* sh_flag) {
  if (a.S == 1) return true;
  const int M = a.M;
  float* mine = a.part + ((size_t)s * M) * a.Np + (size_t)g * kGroupCols;
  for (int idx = threadIdx.x; idx < M * kGroupCols; idx += kThreads) {
    const int r = idx / kGroupCols, c = idx - r * kGroupCols;
    mine[(size_t)r * a.Np + c] = res[r * kResLd + c];
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old = atomicAdd(&a.cnt[g], 1);
    const int last = (old == a.S - 1);
    if (last) atomicExch(&a.cnt[g], 0);
    *sh_flag = last;
  }
  __syncthreads();
  if (!*sh_flag) return false;
  __threadfence();
  for (int idx = threadIdx.x; idx < M * kGroupCols; idx += kThreads) {
    const int r = idx / kGroupCols, c = idx - r * kGroupCols;
    const float* p = a.part + (size_t)r * a.Np + (size_t)g * kGroupCols + c;
    float v = 0.f;
    for (int s2 = 0; s2 < a.S; ++s2) v += p[(size_t)s2 * M * a.Np];
    res[r * kResLd + c] = v;
  }
  __syncthreads();
  return true;
}

template <int EPI>
__device__ void finish(const GemmArgs& a, int g, int s, float* res, float* sh_rowv, int* sh_flag) {
  if (!splitk_finish(a, g, s, res, sh_flag)) return;
  run_epilogue<EPI>(a.e, a.M, g, res, sh_rowv);
}

// ---------------------------------------------------------------- MFMA GEMM
// bf16 weights in MFMA tiles.  MTW = 16-row M tiles per wave.
//   MSPLIT = false: the 4 waves take interleaved k-steps of the same rows
//                   (rows <= 16 * MTW) and are summed in LDS.
//   MSPLIT = true : the 4 waves share every k-step (the B tile is read once
//                   from HBM and served to the others from cache) and each
//                   owns MTW M tiles.
template <int MTW, bool MSPLIT, int NSPLIT, int EPI>
__global__ __launch_bounds__(kThreads) void k_gemm_mfma(GemmArgs a) {
  extern __shared__ float smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = blockIdx.x / a.S, s = blockIdx.x - g * a.S;
  const int ks0 = s * a.kps, ks1 = min(a.KS, ks0 + a.kps);
  const int M = a.M;
  const int mt0 = MSPLIT ? wave * MTW : 0;
  const bf16x8* Wg = reinterpret_cast<const bf16x8*>(a.W) + (size_t)g * a.KS * 256 + lane;

  f32x4 acc[MTW][4];
#pragma unroll
  for (int i = 0; i < MTW; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // rows this lane feeds as the A operand, and whether any is live
  const int arow = lane & 15, akoff = (lane >> 4) * 8;
  const float* xrow[MTW];
  bool xlive[MTW];
#pragma unroll
  for (int i = 0; i < MTW; ++i) {
    const int row = (mt0 + i) * 16 + arow;
    xlive[i] = row < M;
    xrow[i] = a.X + (size_t)(xlive[i] ? row : 0) * a.ldx + akoff;
  }
  const bool wave_live = (mt0 * 16) < M;

  const int kstep = MSPLIT ? 1 : 4;
  int k = MSPLIT ? ks0 : ks0 + wave;

  bf16x8 bA[4], bB[4];
  float4 xA[MTW][2], xB[MTW][2];

#define SV_LOAD(bv, xv, kk)                                                      \
  {                                                                              \
    const bf16x8* wp = Wg + (size_t)(kk) * 256;                                  \
    _Pragma("unroll") for (int t = 0; t < 4; ++t) bv[t] = wp[t * 64];            \
    _Pragma("unroll") for (int i = 0; i < MTW; ++i) {                            \
      if (xlive[i]) {                                                            \
        const float4* xp = reinterpret_cast<const float4*>(xrow[i] + (kk) * kKStep); \
        xv[i][0] = xp[0];                                                        \
        xv[i][1] = xp[1];                                                        \
      } else {                                                                   \
        xv[i][0] = make_float4(0.f, 0.f, 0.f, 0.f);                              \
        xv[i][1] = xv[i][0];                                                     \
      }                                                                          \
    }                                                                            \
  }

#define SV_COMPUTE(bv, xv)                                                       \
  {                                                                              \
    _Pragma("unroll") for (int i = 0; i < MTW; ++i) {                            \
      if ((mt0 + i) * 16 < M) {                                                  \
        const float xs[8] = {xv[i][0].x, xv[i][0].y, xv[i][0].z, xv[i][0].w,      \
                             xv[i][1].x, xv[i][1].y, xv[i][1].z, xv[i][1].w};     \
        bf16x8 av[NSPLIT];                                                       \
        split_bf16x8<NSPLIT>(xs, av);                                            \
        _Pragma("unroll") for (int t = 0; t < 4; ++t) {                          \
          _Pragma("unroll") for (int p = 0; p < NSPLIT; ++p)                     \
            acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[p], bv[t],     \
                                                                acc[i][t], 0, 0, 0); \
        }                                                                        \
      }                                                                          \
    }                                                                            \
  }

  if (wave_live) {
    if (k < ks1) SV_LOAD(bA, xA, k);
    while (k < ks1) {
      const int k2 = k + kstep;
      if (k2 < ks1) SV_LOAD(bB, xB, k2);
      SV_COMPUTE(bA, xA);
      k = k2;
      if (k >= ks1) break;
      const int k3 = k + kstep;
      if (k3 < ks1) SV_LOAD(bA, xA, k3);
      SV_COMPUTE(bB, xB);
      k = k3;
    }
  }
#undef SV_LOAD
#undef SV_COMPUTE

  // C layout of 16x16 MFMA: lane holds rows 4*(lane/16)+j, column lane%16.
  // LDS: MSPLIT -> res [M][kResLd]; k-split -> red [4][16*MTW][kResLd], res [M][kResLd]
  constexpr int R = MTW * 16;
  float* res = MSPLIT ? smem : smem + 4 * R * kResLd;
  const int crow = 4 * (lane >> 4), ccol = lane & 15;
  if constexpr (MSPLIT) {
#pragma unroll
    for (int i = 0; i < MTW; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int row = (mt0 + i) * 16 + crow + j;
          if (row < M) res[row * kResLd + t * 16 + ccol] = acc[i][t][j];
        }
  } else {
    float* red = smem;                 // [4 waves][R][kResLd]
#pragma unroll
    for (int i = 0; i < MTW; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          red[(wave * R + i * 16 + crow + j) * kResLd + t * 16 + ccol] = acc[i][t][j];
    __syncthreads();
    for (int idx = threadIdx.x; idx < M * kGroupCols; idx += kThreads) {
      const int r = idx / kGroupCols, c = idx - r * kGroupCols;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) v += red[(w * R + r) * kResLd + c];
      res[r * kResLd + c] = v;
    }
  }
  __syncthreads();
  __shared__ float sh_rowv[256];
  __shared__ int sh_flag;
  finish<EPI>(a, g, s, res, sh_rowv, &sh_flag);
}

// ---------------------------------------------------------------- vector-FMA GEMM
// Row-major weights (fp32 or bf16).  Lane = (row r = lane / 8 of an 8-row
// step, 8 columns at 8 * (lane % 8)); the 4 waves take interleaved 8-row
// steps of the split's k-range; rows of X are processed 8 at a time.
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

template <typename WT, int EPI>
__global__ __launch_bounds__(kThreads) void k_gemm_fma(GemmArgs a) {
  extern __shared__ float smem[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = blockIdx.x / a.S, s = blockIdx.x - g * a.S;
  const int r0 = s * a.kps * kKStep, r1 = min(a.KS, (s + 1) * a.kps) * kKStep;
  const int M = a.M;
  const int rr = lane >> 3, cg = (lane & 7) * 8;
  const WT* W = reinterpret_cast<const WT*>(a.W) + (size_t)g * kGroupCols + cg;
  float* res = smem;                       // [M][kResLd]
  float* red = smem + M * kResLd;          // [4][8][kResLd]

  for (int m0 = 0; m0 < M; m0 += 8) {
    const int mr = min(8, M - m0);
    float acc[8][8];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[m][j] = 0.f;
    for (int k = r0 + wave * 8 + rr; k < r1; k += 32) {
      float w[8];
      load_w8<WT>(W + (size_t)k * a.Np, w);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        if (m < mr) {
          const float x = a.X[(size_t)(m0 + m) * a.ldx + k];
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[m][j] = fmaf(x, w[j], acc[m][j]);
        }
      }
    }
    // sum the 8 row-lanes that share a column group (lanes differ in bits 3..5)
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float v = acc[m][j];
        v += __shfl_xor(v, 8, kWave);
        v += __shfl_xor(v, 16, kWave);
        v += __shfl_xor(v, 32, kWave);
        acc[m][j] = v;
      }
    if (rr == 0) {
#pragma unroll
      for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int j = 0; j < 8; ++j) red[(wave * 8 + m) * kResLd + cg + j] = acc[m][j];
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < mr * kGroupCols; idx += kThreads) {
      const int m = idx / kGroupCols, c = idx - m * kGroupCols;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) v += red[(w * 8 + m) * kResLd + c];
      res[(m0 + m) * kResLd + c] = v;
    }
    __syncthreads();
  }
  __shared__ float sh_rowv[256];
  __shared__ int sh_flag;
  finish<EPI>(a, g, s, res, sh_rowv, &sh_flag);
}

// ---------------------------------------------------------------- host side
static int mfma_tiles_per_wave(int M) {
  const int mt = (M + 15) / 16;
  if (mt <= 2) return mt;            // k-split inside the work group
  return (mt + 3) / 4;               // rows split over the 4 waves
}

void choose_split(int path, int M, int KS, int G, int& S, int& kps) {
  // Aim for about four work groups per CU over 256 CUs and keep at least
  // two k-steps per wave.
  const int target = 1024;
  const bool msplit = path == PATH_MFMA && (M + 15) / 16 > 2;
  const int min_kps = msplit ? 2 : 8;
  int s = (target + G - 1) / G;
  s = std::min(s, std::max(1, KS / min_kps));
  // partial tiles S*M*Np*4 bytes kept within 1/8 of the weight bytes Kp*Np*2
  const int cap = std::max(1, (2 * KS) / std::max(M, 1));
  s = std::max(1, std::min(s, cap));
  kps = (KS + s - 1) / s;
  S = (KS + kps - 1) / kps;
}

size_t gemm_part_floats(int path, int M, const Mat& m) {
  int S, kps;
  choose_split(path, M, m.Kp / kKStep, m.Np / kGroupCols, S, kps);
  return S > 1 ? (size_t)S * M * m.Np : 0;
}

template <int MTW, bool MSPLIT, int NSPLIT>
static hipError_t launch_mfma_t(int epi, const GemmArgs& a, hipStream_t st) {
  size_t lds = (size_t)a.M * kResLd * sizeof(float);
  if (!MSPLIT) lds += (size_t)4 * MTW * 16 * kResLd * sizeof(float);
  const dim3 grid(a.G * a.S), block(kThreads);
  switch (epi) {
    case EPI_UP: hipLaunchKernelGGL((k_gemm_mfma<MTW, MSPLIT, NSPLIT, EPI_UP>), grid, block, lds, st, a); break;
    case EPI_DOWN: hipLaunchKernelGGL((k_gemm_mfma<MTW, MSPLIT, NSPLIT, EPI_DOWN>), grid, block, lds, st, a); break;
    default: hipLaunchKernelGGL((k_gemm_mfma<MTW, MSPLIT, NSPLIT, EPI_LM>), grid, block, lds, st, a); break;
  }
  return hipGetLastError();
}

template <typename WT>
static hipError_t launch_fma_t(int epi, const GemmArgs& a, hipStream_t st) {
  const size_t lds = ((size_t)a.M * kResLd + 4 * 8 * kResLd) * sizeof(float);
  const dim3 grid(a.G * a.S), block(kThreads);
  switch (epi) {
    case EPI_UP: hipLaunchKernelGGL((k_gemm_fma<WT, EPI_UP>), grid, block, lds, st, a); break;
    case EPI_DOWN: hipLaunchKernelGGL((k_gemm_fma<WT, EPI_DOWN>), grid, block, lds, st, a); break;
    default: hipLaunchKernelGGL((k_gemm_fma<WT, EPI_LM>), grid, block, lds, st, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(int path, int epi, const GemmArgs& a, hipStream_t st) {
  if (path == PATH_FMA_F32) return launch_fma_t<float>(epi, a, st);
  if (path == PATH_FMA_BF16) return launch_fma_t<uint16_t>(epi, a, st);
  const int mtw = mfma_tiles_per_wave(a.M);
  const bool msplit = (a.M + 15) / 16 > 2;
  if (!msplit) {
    if (mtw == 1) return launch_mfma_t<1, false, 3>(epi, a, st);
    return launch_mfma_t<2, false, 3>(epi, a, st);
  }
  switch (mtw) {
    case 1: return launch_mfma_t<1, true, 3>(epi, a, st);
    case 2: return launch_mfma_t<2, true, 3>(epi, a, st);
    case 3: return launch_mfma_t<3, true, 3>(epi, a, st);
    default: return launch_mfma_t<4, true, 3>(epi, a, st);
  }
}

}  // namespace sv
