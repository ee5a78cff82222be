// Host-side structures and kernel launchers shared by the library's sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "common.h"

namespace sv {

enum WeightFormat { FMT_ROWMAJOR_F32 = 0, FMT_ROWMAJOR_BF16 = 1, FMT_MFMA_BF16 = 2 };

// One weight matrix W[K][N] as the library holds it.  Every layout is
// zero-padded to Kp = roundup(K, 32) rows and Np = roundup(N, 64) columns.
//   row-major: element (k, n) at k * Np + n
//   MFMA tiles, in column blocks of nt 16-column tiles: 16-byte chunks at
//     ((b * KS + s) * nt + t) * 64 + lane holding
//     W[32 s + 8 (lane / 16) + j][16 (b * nt + t) + lane % 16], j = 0..7,
//     where b = column block, s = k-step of 32 rows, KS = Kp / 32, t = tile
//     in the block: exactly the B operand of one 16x16x32 bf16 MFMA per
//     (b, s, t), and the whole of one column block is one contiguous span,
//     read by the one work group that owns it.
struct Mat {
  int K = 0, N = 0, Kp = 0, Np = 0;
  int nt = 4;                 // MFMA layout: 16-column tiles per column block
  void* rowmajor = nullptr;   // FMT_ROWMAJOR_F32 / _BF16
  void* mfma = nullptr;       // FMT_MFMA_BF16
};

// Column block width (in 16-column tiles) of the MFMA layout for N columns:
// the widest of 4, 2, 1 that still gives every CU a work group.
int mfma_block_tiles(int Np);

// Epilogue of a GEMM, run by the work group that owns the columns.
enum EpiKind { EPI_UP = 0, EPI_DOWN = 1, EPI_LM = 2 };

struct EpiArgs {
  int kind = EPI_UP;
  float* out = nullptr;       // act (UP) / h (DOWN) / logits (LM), row stride ldo
  int ldo = 0;
  int N = 0;                  // valid columns
  // UP: 1 / rms from per-16-column sums of squares of the block input
  const float* ss_in = nullptr;
  int ss_ld = 0, ss_n = 0;
  float inv_d = 0.f, eps = 0.f;
  float* rms = nullptr;       // UP, wide path: 1 / rms of every row of the pass,
                              // written by the GEMM, read by its epilogue
  // DOWN: next block's normalised input and its sums of squares
  float* xg = nullptr;
  const float* gain_next = nullptr;   // null: last block
  float* ss_out = nullptr;
  // LM: per-16-column-subtile softmax / argmax statistics of p and of q
  float* pst = nullptr;       // [rows][G][2]
  int* pidx = nullptr;        // [rows][G]   (greedy)
  float* qst = nullptr;       // [B*gamma][G][2]
  const float* q = nullptr;   // [B][gamma][V]
  int G = 0;                  // row stride of the statistics (units, even)
  int G1 = 1, gamma = 0, V = 0;
  int row0 = 0;               // global index of this launch's first row
  int tmode = 0;              // 0 greedy, 1 T == 1, 2 general T
  float invT = 1.f;
  // the output again as split bf16 A fragments for the next GEMM (xs_index
  // order, xs_ks k-steps; null when that GEMM is not an MFMA one): UP
  // writes act, DOWN the next block's normalised input or, after the last
  // block, h for the LM head
  uint16_t* xs = nullptr;
  int xs_ks = 0;
  bool xs_stack = false;      // stacked packing (xs_index)
  bool xs_two = false;        // two-term split (split2_bf16)
};

struct GemmArgs {
  const float* X = nullptr;   // [M][ldx] fp32, columns >= K are zero (FMA path)
  const void* XS = nullptr;   // X as split bf16 A fragments, KS + 1 k-steps (MFMA path)
  int ldx = 0, M = 0, K = 0;
  const void* W = nullptr;
  int Np = 0, KS = 0;         // KS = Kp / 32
  EpiArgs e;
};

// Waves of a vector-FMA GEMM work group (k_gemm_fma).
constexpr int kFmaWaves = 8;

// Launch plan of one GEMM (chosen on the host by plan_gemm).
enum GemmPath { PATH_FMA_F32 = 0, PATH_FMA_BF16 = 1, PATH_MFMA = 2 };

struct GemmPlan {
  int path = PATH_MFMA;
  int mtw = 1, mg = 1, kg = 1;   // M tiles per wave, row groups, k-groups
  int nt = 4;                    // 16-column tiles per work group
  bool stack = false;            // stacked activation packing (MFMA)
  bool two = false;              // stacked: two terms of eight rows per tile
  int blocks = 0;                // work groups
  size_t lds = 0;                // dynamic LDS bytes
};

// The MFMA path packs the split activations of up to 8 rows stacked (one
// five-row tile of three terms up to 5 rows, one eight-row tile of two terms
// for 6 to 8, or two five-row tiles of three with the exact split; one
// fragment per k-step each); more rows use the plain packing on the wide
// GEMM (measured: B = 1 passes of 9 and 10 rows 5% faster there on the mid
// model and 7% on the large one than in two stacked tiles).
inline bool xs_stacked(int M) { return M <= kStackRows2; }

// Bytes of one split-activation buffer of M rows and ks k-steps (plus the
// all-zero step): one 1 KiB fragment per row tile and k-step stacked (sized
// for five-row tiles, which the eight-row tiles never exceed), three plain.
inline size_t xs_bytes(int M, int ks) {
  return xs_stacked(M) ? (size_t)((M + kStackRows - 1) / kStackRows) * (ks + 1) * 1024
                       : (size_t)((M + 15) / 16) * (ks + 1) * 3 * 1024;
}

GemmPlan plan_gemm(int path, int M, const Mat& m, bool stack, bool two);

// Wide MFMA GEMM (plain packing): work groups of 8 column tiles with the
// activations staged in LDS, K split over S slices when the column blocks
// alone cannot fill the chip.
struct WidePlan {
  int MT = 0, mtw = 0, ntc = 0, mg = 0, cg = 0;
  int terms = 3;              // bf16 terms per activation the GEMM reads
  int colblocks = 0, S = 1, ks_slice = 0;
  size_t lds = 0;
};
struct WideArgs {
  const void* XS = nullptr;   // split activations, plain packing
  const void* W = nullptr;    // MFMA weight tiles
  int M = 0, MT = 0, KS = 0;
  int nt = 1, tiles = 0;      // layout column-block width (tiles) and tiles of Np
  int ks_slice = 0, S = 1;
  float* P = nullptr;         // [S][M][ldp] fp32 partial sums
  int ldp = 0;
  size_t slice_stride = 0;    // floats between slices
  bool fuse_lm = false;       // LM head in one slice: the GEMM writes the
                              // logits and unit statistics, P is unused
};
WidePlan plan_wide(int M, const Mat& m, bool two_term);
// Row counts the wide GEMM serves: the plain packing up to one 224-row chunk.
inline bool wide_rows(int M) { return !xs_stacked(M) && M <= 224; }
// The GEMM (timed by e0 / e1 when given) and then its epilogue kernel; an
// LM head in one K slice runs its epilogue inside the GEMM.
hipError_t launch_wide(const WidePlan& p, const WideArgs& a, const EpiArgs& e, hipStream_t st,
                       hipEvent_t e0, hipEvent_t e1);
// e0 / e1: null, or events that take the launch's start and end timestamps.
hipError_t launch_gemm(const GemmPlan& p, const GemmArgs& a, hipStream_t st, hipEvent_t e0,
                       hipEvent_t e1);

// Sampling-side launchers (sample.hip).
struct SampleArgs {
  int B = 0, gamma = 0, V = 0, G = 0, Gu = 0;   // G: statistics row stride, Gu: units
  int M = 0;                  // B * (gamma + 1)
  const float* logits = nullptr; int ldl = 0;
  const float* q = nullptr;
  const int* draft = nullptr;
  float T = 1.f, invT = 1.f, top_p = 1.f;
  int tmode = 0;
  uint64_t seed = 0;
  int* n_acc = nullptr; int* emitted = nullptr;
  float* pst = nullptr; int* pidx = nullptr; float* qst = nullptr;   // G subtiles per row
  float* rowinfo = nullptr;   // [M + B*gamma][8]
  int* dec = nullptr;         // [B][4]
  double* csum = nullptr;     // [B][nch][2]
  int nch = 0;
  float* p_out = nullptr; float* q_out = nullptr;   // debug dumps
};

// Copies hidden into h, forms xg = h * gain0 and its per-16-column sums of
// squares; with xs0 non-null also writes the first GEMM's split input (xg,
// or h when there is no MLP block) and clears the zero k-step of each of
// the split buffers xs0 (ks0 k-steps) and xs1 (ks1 k-steps), packed as
// xs_stacked(M) says, in two terms when `two`.
hipError_t launch_prep(float* h, float* xg, float* ss, int ss_ld, const float* hidden,
                       const float* gain0, int M, int d, int ld, uint16_t* xs0, int ks0,
                       uint16_t* xs1, int ks1, bool two, hipStream_t st);
hipError_t launch_tile_stats(const SampleArgs& a, hipStream_t st);
hipError_t launch_sampling(const SampleArgs& a, hipStream_t st);
hipError_t launch_dump_probs(const SampleArgs& a, hipStream_t st);
// Greedy tree walk after a T = 0 pass over B (n + 1) rows (a.gamma = n
// nodes): per-row argmax, then the walk per sequence.
hipError_t launch_tree_walk(const SampleArgs& a, const int* parent, const int* tokens, int* path,
                            hipStream_t st);

// Weight conversion launchers (pack.hip).
hipError_t launch_pack_mfma(const void* src, int src_dtype, int K, int N, void* dst, int Kp,
                            int Np, int nt, hipStream_t st);
hipError_t launch_copy_rowmajor(const void* src, int src_dtype, int K, int N, void* dst,
                                int dst_dtype, int Kp, int Np, hipStream_t st);
hipError_t launch_vec_to_f32(const void* src, int src_dtype, int n, float* dst, hipStream_t st);

// Streaming read of `bytes` (a multiple of 16, 16-byte aligned) from src
// (probe.hip).
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t key, uint32_t* sink,
                              hipStream_t st);

constexpr int kResampleChunk = 1024;   // elements per resample chunk

}  // namespace sv
