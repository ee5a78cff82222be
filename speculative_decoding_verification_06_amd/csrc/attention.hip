// Attention of a verification pass's new rows over a KV-cached prefix, and
// the commit of the accepted rows ("Speculative Decoding: Speeding Sequential
// Generation", aicomputerinstitute.com, Constructing the Tree Attention Mask
// in Code; "Build a Speculative Decoding Engine to Cut LLM Latency by 3x",
// scalablesystem.dev, KV Cache Management for Dual Models, Rollback
// Protocol).
//
// Cache layout [B][Hkv][max_seq][HD] bf16: one key's (or value's) head
// dimension is one contiguous 2*HD-byte row.  New row i of sequence b is the
// query q[b][i][h][:] (fp32); its key and value sit at slot L_b + i.  Row i
// sees slots 0 .. L_b - 1 and the new slots of itself and its ancestors.
//
// Work decomposition: a work group of 4 waves owns (sequence, KV head, group
// of up to kRows query rows: new rows x the H / Hkv query heads sharing the
// KV head, split of the keys); each wave streams its own tiles of 64 keys,
// so every key and value byte of a split is read once for all query rows of
// the group (the weight-streaming idea of the GEMMs, applied to the cache).
// Scores: lane = key, the lane's key row in registers, the group's query
// rows read with wave-uniform addresses.  P V: lane = 2 (HD 128) or 1 (HD
// 64) head dimensions, one coalesced value row per key, the tile's
// probabilities through LDS.  Online softmax per row; every wave writes its
// partial (max, sum, unnormalised output), and a second kernel merges the
// partials in a fixed order, so results are run-to-run identical.

#include <algorithm>
#include <climits>
#include <cmath>

#include "common.h"
#include "internal.h"
#include "specverify.h"

#pragma clang fp contract(off)

namespace sv {

constexpr int kAttnWaves = 4;
constexpr int kAttnThreads = kAttnWaves * kWave;
constexpr int kAttnRows = 32;      // query rows of a work group
constexpr int kAttnTile = 64;      // keys per wave tile

struct AttnArgs {
  int B, n_new, H, Hkv, G, max_seq, R, RG, S;   // R = n_new * G rows, RG row groups, S splits
  const float* q;            // [B][n_new][H][HD]
  const uint16_t* k;         // [B][Hkv][max_seq][HD]
  const uint16_t* v;
  const int* cache_len;      // [B]
  const int* parent;         // [B][n_new] or null (chain)
  float scale;
  float* part_o;             // [B][Hkv][RG][S * waves][kAttnRows][HD]
  float* part_ml;            // [B][Hkv][RG][S * waves][kAttnRows][2]
  float* out;                // [B][n_new][H][HD]
};

__device__ __forceinline__ int attn_len(const AttnArgs& a, int b) {
  // committed length, clamped so the new slots stay inside the cache
  const int L = a.cache_len[b];
  return L < 0 ? 0 : (L > a.max_seq - a.n_new ? a.max_seq - a.n_new : L);
}

template <int HD>
__global__ __launch_bounds__(kAttnThreads) void k_decode_attn(AttnArgs a) {
  constexpr int DPL = HD / kWave;                  // head dimensions per lane in P V
  constexpr int KCH = HD / 8;                      // 16-byte chunks of one key row
  __shared__ uint64_t anc[64];                     // visible new rows of each new row
  __shared__ float pbuf[kAttnWaves][kAttnRows][kAttnTile];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.x, rg = blockIdx.y % a.RG, kvh = blockIdx.y / a.RG, b = blockIdx.z;
  const int L = attn_len(a, b), T = L + a.n_new;
  const int r0 = rg * kAttnRows, nr = min(kAttnRows, a.R - r0);

  if (threadIdx.x == 0) {
    uint64_t m = 0;
    for (int i = 0; i < a.n_new; ++i) {
      int p = a.parent ? a.parent[(size_t)b * a.n_new + i] : i - 1;
      if (p < -1 || p >= i) p = -1;                // a bad parent sees no other new row
      m = (p >= 0 ? anc[p] : 0ull) | (1ull << i);
      anc[i] = m;
    }
  }
  __syncthreads();

  // this wave's keys: split `split` of S, quarter `wave` of it, in tiles
  const int per_split = (((T + a.S - 1) / a.S) + kAttnTile - 1) / kAttnTile * kAttnTile;
  const int s0 = min(T, split * per_split), s1 = min(T, s0 + per_split);
  const int per_wave = (((s1 - s0) + kAttnWaves - 1) / kAttnWaves + kAttnTile - 1) / kAttnTile * kAttnTile;
  const int w0 = min(s1, s0 + wave * per_wave), w1 = min(s1, w0 + per_wave);

  const uint16_t* K = a.k + ((size_t)b * a.Hkv + kvh) * a.max_seq * HD;
  const uint16_t* V = a.v + ((size_t)b * a.Hkv + kvh) * a.max_seq * HD;
  // query row r of the group: new row i = r / G, head kvh * G + r % G
  auto qrow = [&](int r) -> const float* {
    const int rr = r0 + r, i = rr / a.G, h = kvh * a.G + rr % a.G;
    return a.q + (((size_t)b * a.n_new + i) * a.H + h) * HD;
  };

  float m[kAttnRows], l[kAttnRows], o[kAttnRows][DPL];
#pragma unroll
  for (int r = 0; r < kAttnRows; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.f;
#pragma unroll
    for (int j = 0; j < DPL; ++j) o[r][j] = 0.f;
  }

  for (int t = w0; t < w1; t += kAttnTile) {
    const int key = t + lane;
    const bool kv_ok = key < w1;
    const int kc = kv_ok ? key : w1 - 1;           // in-bounds row for idle lanes
    // the lane's key row, all chunks in flight
    u32x4 kr[KCH];
    const u32x4* kp = reinterpret_cast<const u32x4*>(K + (size_t)kc * HD);
#pragma unroll
    for (int c = 0; c < KCH; ++c) kr[c] = kp[c];
    float s[kAttnRows];
#pragma unroll
    for (int r = 0; r < kAttnRows; ++r) s[r] = 0.f;
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      float kf[8];
      kf[0] = bf16_lo(kr[c].x); kf[1] = bf16_hi(kr[c].x); kf[2] = bf16_lo(kr[c].y); kf[3] = bf16_hi(kr[c].y);
      kf[4] = bf16_lo(kr[c].z); kf[5] = bf16_hi(kr[c].z); kf[6] = bf16_lo(kr[c].w); kf[7] = bf16_hi(kr[c].w);
#pragma unroll
      for (int r = 0; r < kAttnRows; ++r) {
        if (r < nr) {
          const float* qp = qrow(r) + c * 8;
#pragma unroll
          for (int j = 0; j < 8; ++j) s[r] = fmaf(qp[j], kf[j], s[r]);
        }
      }
    }
    // mask, scale, online softmax per row; probabilities to LDS
    const int jn = key - L;                         // new slot index, when >= 0
#pragma unroll
    for (int r = 0; r < kAttnRows; ++r) {
      if (r >= nr) continue;
      const int i = (r0 + r) / a.G;
      const bool vis = kv_ok && (jn < 0 || ((anc[i] >> jn) & 1ull));
      const float sc = vis ? s[r] * a.scale : -INFINITY;
      const float mt = wave_max(sc);
      const float mn = fmaxf(m[r], mt);
      float p = 0.f, corr = 1.f;
      if (mn > -INFINITY) {
        p = vis ? expf(sc - mn) : 0.f;
        corr = m[r] > -INFINITY ? expf(m[r] - mn) : 0.f;
      }
      l[r] = l[r] * corr + wave_sum(p);
      m[r] = mn;
#pragma unroll
      for (int j = 0; j < DPL; ++j) o[r][j] *= corr;
      pbuf[wave][r][lane] = p;
    }
    // the tile's probabilities are read by every lane of the wave below
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // P V: lane owns dimensions DPL * lane .. + DPL - 1; keys of the tile in
    // batches of 16 with their value loads in flight
    const int nk = min(kAttnTile, w1 - t);
    for (int k0 = 0; k0 < nk; k0 += 16) {
      float vv[16][DPL];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int kk = min(k0 + u, nk - 1);
        const uint16_t* vp = V + (size_t)(t + kk) * HD + DPL * lane;
        if constexpr (DPL == 2) {
          const uint32_t w2 = *reinterpret_cast<const uint32_t*>(vp);
          vv[u][0] = bf16_lo(w2);
          vv[u][1] = bf16_hi(w2);
        } else {
          vv[u][0] = __uint_as_float((uint32_t)vp[0] << 16);
        }
      }
#pragma unroll
      for (int r = 0; r < kAttnRows; ++r) {
        if (r >= nr) continue;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const float p = k0 + u < nk ? pbuf[wave][r][k0 + u] : 0.f;
#pragma unroll
          for (int j = 0; j < DPL; ++j) o[r][j] = fmaf(p, vv[u][j], o[r][j]);
        }
      }
    }
    // every lane has read the tile's probabilities before the next tile's
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // this wave's partial state
  const size_t unit = (((size_t)b * a.Hkv + kvh) * a.RG + rg) * (size_t)(a.S * kAttnWaves) +
                      (size_t)split * kAttnWaves + wave;
  float* po = a.part_o + unit * kAttnRows * HD;
  float* pml = a.part_ml + unit * kAttnRows * 2;
#pragma unroll
  for (int r = 0; r < kAttnRows; ++r) {
    if (r >= nr) continue;
#pragma unroll
    for (int j = 0; j < DPL; ++j) po[r * HD + DPL * lane + j] = o[r][j];
    if (lane == 0) { pml[2 * r] = m[r]; pml[2 * r + 1] = l[r]; }
  }
}

// Merge the S * waves partial states of every query row in order: out =
// sum_p o_p exp(m_p - M) / sum_p l_p exp(m_p - M), M the largest m_p.
template <int HD>
__global__ __launch_bounds__(HD) void k_attn_combine(AttnArgs a) {
  const int d = threadIdx.x, r = blockIdx.x, rg = blockIdx.y % a.RG, kvh = blockIdx.y / a.RG,
            b = blockIdx.z;
  const int rr = rg * kAttnRows + r;
  if (rr >= a.R) return;
  const int P = a.S * kAttnWaves;
  const size_t unit0 = (((size_t)b * a.Hkv + kvh) * a.RG + rg) * (size_t)P;
  float M = -INFINITY;
  for (int p = 0; p < P; ++p) M = fmaxf(M, a.part_ml[((unit0 + p) * kAttnRows + r) * 2]);
  float num = 0.f, den = 0.f;
  if (M > -INFINITY) {
    for (int p = 0; p < P; ++p) {
      const float mp = a.part_ml[((unit0 + p) * kAttnRows + r) * 2];
      if (mp == -INFINITY) continue;
      const float w = expf(mp - M);
      den += a.part_ml[((unit0 + p) * kAttnRows + r) * 2 + 1] * w;
      num += a.part_o[((unit0 + p) * kAttnRows + r) * HD + d] * w;
    }
  }
  const int i = rr / a.G, h = kvh * a.G + rr % a.G;
  a.out[(((size_t)b * a.n_new + i) * a.H + h) * HD + d] = den > 0.f ? num / den : 0.f;
}

// ---------------------------------------------------------------- commit
// Tree commit: the accepted path's rows (node j = new row j + 1) gathered to
// slots L + 1 .. L + n, for every KV head; all rows are read before any is
// written.  One work group per (KV head, sequence).
template <int HD>
__global__ __launch_bounds__(256) void k_kv_gather(int B, int n_new, int Hkv, int max_seq,
                                                   uint16_t* k, uint16_t* v, const int* cache_len,
                                                   const int* n_accepted, const int* path) {
  __shared__ uint32_t rows[2][64][HD / 2];
  const int kvh = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int n = n_accepted[b];
  if (n <= 0 || n > n_new - 1) return;
  int L = cache_len[b];
  L = L < 0 ? 0 : (L > max_seq - n_new ? max_seq - n_new : L);
  const size_t base = ((size_t)b * Hkv + kvh) * max_seq;
  uint32_t* K32 = reinterpret_cast<uint32_t*>(k + base * HD);
  uint32_t* V32 = reinterpret_cast<uint32_t*>(v + base * HD);
  constexpr int W = HD / 2;
  for (int x = tid; x < n * W; x += 256) {
    const int kk = x / W, c = x - kk * W;
    int node = path[(size_t)b * (n_new - 1) + kk];
    node = node < 0 ? 0 : (node > n_new - 2 ? n_new - 2 : node);
    const size_t src = (size_t)(L + 1 + node) * W + c;
    rows[0][kk][c] = K32[src];
    rows[1][kk][c] = V32[src];
  }
  __syncthreads();
  for (int x = tid; x < n * W; x += 256) {
    const int kk = x / W, c = x - kk * W;
    const size_t dst = (size_t)(L + 1 + kk) * W + c;
    K32[dst] = rows[0][kk][c];
    V32[dst] = rows[1][kk][c];
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
  int R = 0, RG = 0, S = 0;
  size_t o_off = 0, ml_off = 0, total = 0;
};

AttnShape attn_shape(int B, int n_new, int H, int Hkv, int hd, int max_seq) {
  AttnShape s;
  const int G = H / Hkv;
  s.R = n_new * G;
  s.RG = (s.R + kAttnRows - 1) / kAttnRows;
  // enough work groups to cover the CUs about four times over, each split
  // at least one tile per wave
  const int groups = B * Hkv * s.RG;
  const int want = (1024 + groups - 1) / groups;
  const int most = std::max(1, max_seq / (kAttnTile * kAttnWaves));
  s.S = std::max(1, std::min(want, most));
  const size_t units = (size_t)groups * s.S * kAttnWaves;
  s.o_off = 0;
  s.ml_off = (units * kAttnRows * hd * sizeof(float) + 255) & ~(size_t)255;
  s.total = s.ml_off + ((units * kAttnRows * 2 * sizeof(float) + 255) & ~(size_t)255);
  return s;
}

bool attn_args_ok(int B, int n_new, int H, int Hkv, int hd, int max_seq) {
  return B >= 1 && n_new >= 1 && n_new <= 64 && Hkv >= 1 && H >= Hkv && H % Hkv == 0 &&
         (hd == 64 || hd == 128) && max_seq >= n_new;
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
  a.q = q; a.k = k_cache; a.v = v_cache; a.cache_len = cache_len; a.parent = parent;
  a.scale = scale; a.out = out;
  a.part_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + s.o_off);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + s.ml_off);
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const dim3 grid(s.S, Hkv * s.RG, B);
  if (head_dim == 128) {
    hipLaunchKernelGGL(k_decode_attn<128>, grid, dim3(kAttnThreads), 0, st, a);
    hipLaunchKernelGGL(k_attn_combine<128>, dim3(kAttnRows, Hkv * s.RG, B), dim3(128), 0, st, a);
  } else {
    hipLaunchKernelGGL(k_decode_attn<64>, grid, dim3(kAttnThreads), 0, st, a);
    hipLaunchKernelGGL(k_attn_combine<64>, dim3(kAttnRows, Hkv * s.RG, B), dim3(64), 0, st, a);
  }
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
