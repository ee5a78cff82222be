// Host policy around the verification step ("Build a Speculative Decoding
// Engine to Cut LLM Latency by 3x", scalablesystem.dev):
//
//   gamma controller : per-sequence rolling window of (accepted, rejected)
//                      counts, 20 steps; from 5 steps on, gamma is the value
//                      in [gamma_min, gamma_max] that maximises
//                      E(gamma) / (gamma t_draft + t_target(gamma)),
//                      E(gamma) = (1 - alpha^(gamma+1)) / (1 - alpha)
//                      (Dynamic Gamma Controller), with t_target a table of
//                      measured verification times per gamma
//   repack           : after a step, rows accepted different counts (Batch-
//                      Level Speculation): the emitted tokens packed end to
//                      end with row offsets, the committed lengths advanced,
//                      the padded width and waste of one padded batch, and
//                      the sequences binned by emitted count (a stable
//                      counting sort) for micro-batches.  One work group on
//                      the device, so it runs after the verification step on
//                      the same stream with no host round trip.

#include <cmath>
#include <new>
#include <vector>

#include "common.h"
#include "internal.h"
#include "specverify.h"

namespace sv {

// ---------------------------------------------------------------- repack
constexpr int kRepackThreads = 1024;
constexpr int kRepackWaves = kRepackThreads / kWave;
constexpr int kRepackMaxBins = 256;      // emitted counts 0 .. gamma + 1

__global__ __launch_bounds__(kRepackThreads) void k_repack(int B, int G1, const int* n_acc,
                                                           const int* emitted, int* committed,
                                                           int* tokens, int* offsets, int* order,
                                                           int* bin_offsets, int* stats) {
  __shared__ int wave_bin[kRepackWaves][kRepackMaxBins];   // per-wave bin counts of a chunk
  __shared__ int bin_base[kRepackMaxBins];                 // running start of each bin
  __shared__ int wave_sum[kRepackWaves];
  __shared__ int sh_width, sh_total;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nbins = G1 + 1;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  // bin sizes over the whole batch, then their exclusive prefix
  for (int c = tid; c < nbins; c += kRepackThreads) bin_base[c] = 0;
  if (tid == 0) { sh_width = 0; sh_total = 0; }
  __syncthreads();
  // a row emitted n + 1 tokens when 0 <= n < G1; any other n (a refused
  // row, -1) emitted none
  for (int b = tid; b < B; b += kRepackThreads) {
    const int n = n_acc[b];
    const int cnt = n >= 0 && n < G1 ? n + 1 : 0;
    atomicAdd(&bin_base[cnt], 1);
    atomicMax(&sh_width, cnt);
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int c = 0; c < nbins; ++c) {
      const int x = bin_base[c];
      bin_base[c] = run;
      bin_offsets[c] = run;
      run += x;
    }
    bin_offsets[nbins] = B;
  }
  __syncthreads();

  // chunks of kRepackThreads sequences in order: offsets by a block scan,
  // bin ranks by per-wave ballots (stable: wave order, then lane order)
  int carry = 0;
  for (int b0 = 0; b0 < B; b0 += kRepackThreads) {
    const int b = b0 + tid;
    const bool live = b < B;
    const int n = live ? n_acc[b] : -1;
    const int cnt = live && n >= 0 && n < G1 ? n + 1 : 0;
    // exclusive scan of cnt over the chunk
    int inc = cnt;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(inc, o, kWave);
      if (lane >= o) inc += y;
    }
    if (lane == kWave - 1) wave_sum[wave] = inc;
    // rank among the wave's lanes of the same bin
    int rank = 0;
    for (int c = 0; c < nbins; ++c) {
      const uint64_t m = __ballot(live && cnt == c);
      if (live && cnt == c) rank = __popcll(m & below);
      if (lane == 0) wave_bin[wave][c] = __popcll(m);
    }
    __syncthreads();
    int base = carry;
    for (int w = 0; w < wave; ++w) base += wave_sum[w];
    const int off = base + inc - cnt;
    int before = 0;                      // same-bin sequences of earlier waves in the chunk
    for (int w = 0; w < wave; ++w) before += wave_bin[w][cnt];
    if (live) {
      offsets[b] = off;
      committed[b] += cnt;
      for (int i = 0; i < cnt; ++i) tokens[off + i] = emitted[(size_t)b * G1 + i];
      order[bin_base[cnt] + before + rank] = b;
    }
    __syncthreads();
    if (tid == 0) {
      for (int w = 0; w < kRepackWaves; ++w) carry += wave_sum[w];
      for (int c = 0; c < nbins; ++c) {
        int s = 0;
        for (int w = 0; w < kRepackWaves; ++w) s += wave_bin[w][c];
        bin_base[c] += s;
      }
      sh_total = carry;
    }
    __syncthreads();
    carry = sh_total;
  }
  if (tid == 0) {
    offsets[B] = carry;
    stats[0] = sh_width;
    stats[1] = B * sh_width - carry;
  }
}

}  // namespace sv

using namespace sv;

// ---------------------------------------------------------------- gamma controller
struct spec_gamma_ctl {
  static constexpr int kWindow = 20;
  static constexpr int kMinSteps = 5;
  static constexpr double kDefaultAlpha = 0.80;
  int n_seq = 0, gmin = 0, gmax = 0;
  double draft_ms = 0.0;
  std::vector<double> target_ms;        // [gmax + 1]
  std::vector<int> gamma;               // [n_seq]
  std::vector<int> acc, rej, len, head; // [n_seq]: window sums, fill, next slot
  std::vector<int> ring_a, ring_r;      // [n_seq * kWindow]: the window's steps

  double alpha(int s) const {
    if (len[s] == 0) return kDefaultAlpha;
    const int tot = acc[s] + rej[s];
    return (double)acc[s] / (double)(tot > 0 ? tot : 1);
  }
  double expected(double a, int g) const {
    if (a >= 1.0) return (double)(g + 1);
    return (1.0 - std::pow(a, g + 1)) / (1.0 - a);
  }
  int optimal(double a) const {
    int best = gmin;
    double best_rate = -1.0;
    for (int g = gmin; g <= gmax; ++g) {
      const double rate = expected(a, g) / ((double)g * draft_ms + target_ms[g]);
      if (rate > best_rate) { best = g; best_rate = rate; }
    }
    return best;
  }
  void record(int s, int a, int r) {
    const int slot = s * kWindow + head[s];
    if (len[s] == kWindow) { acc[s] -= ring_a[slot]; rej[s] -= ring_r[slot]; }
    else ++len[s];
    ring_a[slot] = a;
    ring_r[slot] = r;
    acc[s] += a;
    rej[s] += r;
    head[s] = (head[s] + 1) % kWindow;
  }
};

extern "C" {

spec_status spec_gamma_ctl_create(int32_t n_seq, int32_t gamma_min, int32_t gamma_max,
                                  int32_t gamma_init, double draft_ms_per_token,
                                  const double* target_ms, spec_gamma_ctl_t* out) {
  if (!out || n_seq < 1 || gamma_min < 0 || gamma_init < gamma_min || gamma_max < gamma_init ||
      !target_ms || !(draft_ms_per_token >= 0.0) || !std::isfinite(draft_ms_per_token))
    return SPEC_EINVAL;
  for (int g = gamma_min; g <= gamma_max; ++g)
    if (!(target_ms[g] > 0.0) || !std::isfinite(target_ms[g])) return SPEC_EINVAL;
  spec_gamma_ctl* c = new (std::nothrow) spec_gamma_ctl;
  if (!c) return SPEC_ENOMEM;
  c->n_seq = n_seq; c->gmin = gamma_min; c->gmax = gamma_max; c->draft_ms = draft_ms_per_token;
  c->target_ms.assign(target_ms, target_ms + gamma_max + 1);
  c->gamma.assign(n_seq, gamma_init);
  c->acc.assign(n_seq, 0); c->rej.assign(n_seq, 0); c->len.assign(n_seq, 0); c->head.assign(n_seq, 0);
  c->ring_a.assign((size_t)n_seq * spec_gamma_ctl::kWindow, 0);
  c->ring_r.assign((size_t)n_seq * spec_gamma_ctl::kWindow, 0);
  *out = c;
  return SPEC_OK;
}

spec_status spec_gamma_ctl_destroy(spec_gamma_ctl_t c) {
  delete c;
  return SPEC_OK;
}

spec_status spec_gamma_ctl_update(spec_gamma_ctl_t c, const int32_t* n_accepted,
                                  const int32_t* gamma_used, int32_t* gamma_next) {
  if (!c || !n_accepted || !gamma_used || !gamma_next) return SPEC_EINVAL;
  for (int s = 0; s < c->n_seq; ++s)
    if (n_accepted[s] > gamma_used[s] || gamma_used[s] < 0) return SPEC_EINVAL;
  for (int s = 0; s < c->n_seq; ++s) {
    if (n_accepted[s] >= 0) {
      c->record(s, n_accepted[s], gamma_used[s] - n_accepted[s]);
      if (c->len[s] >= spec_gamma_ctl::kMinSteps) c->gamma[s] = c->optimal(c->alpha(s));
    }
    gamma_next[s] = c->gamma[s];
  }
  return SPEC_OK;
}

double spec_gamma_ctl_alpha(spec_gamma_ctl_t c, int32_t seq) {
  if (!c || seq < 0 || seq >= c->n_seq) return -1.0;
  return c->alpha(seq);
}

int32_t spec_gamma_ctl_optimal(spec_gamma_ctl_t c, double alpha) {
  if (!c || !(alpha >= 0.0 && alpha <= 1.0)) return -1;
  return c->optimal(alpha);
}

spec_status spec_repack(int32_t B, int32_t gamma, const int32_t* n_accepted,
                        const int32_t* emitted, int32_t* committed, int32_t* tokens,
                        int32_t* offsets, int32_t* order, int32_t* bin_offsets, int32_t* stats,
                        void* stream) {
  if (B < 1 || gamma < 0 || gamma + 2 > kRepackMaxBins || !n_accepted || !emitted || !committed ||
      !tokens || !offsets || !order || !bin_offsets || !stats)
    return SPEC_EINVAL;
  if ((int64_t)B * (gamma + 1) > INT32_MAX) return SPEC_EINVAL;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_repack, dim3(1), dim3(kRepackThreads), 0, static_cast<hipStream_t>(stream),
                     B, gamma + 1, n_accepted, emitted, committed, tokens, offsets, order,
                     bin_offsets, stats);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

}  // extern "C"
