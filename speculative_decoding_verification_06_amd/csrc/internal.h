// Host-side structures and kernel launchers shared by the library's sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

namespace sv {

enum WeightFormat { FMT_ROWMAJOR_F32 = 0, FMT_ROWMAJOR_BF16 = 1, FMT_MFMA_BF16 = 2 };

// One weight matrix W[K][N] as the library holds it.  Every layout is
// zero-padded to Kp = roundup(K, 32) rows and Np = roundup(N, 64) columns.
//   row-major: element (k, n) at k * Np + n
//   MFMA tiles: 16-byte chunks at ((g * KS + s) * 4 + t) * 64 + lane holding
//     W[32 s + 8 (lane / 16) + j][64 g + 16 t + lane % 16], j = 0..7, where
//     g = column group of 64, s = k-step of 32 rows, KS = Kp / 32: exactly the
//     B operand of one 16x16x32 bf16 MFMA per (g, s, t), and one work
//     group's k-range of a column group is one contiguous span.
struct Mat {
  int K = 0, N = 0, Kp = 0, Np = 0;
  void* rowmajor = nullptr;   // FMT_ROWMAJOR_F32 / _BF16
  void* mfma = nullptr;       // FMT_MFMA_BF16
};

// Epilogue of a split-K GEMM, run by the last work group of each column group.
enum EpiKind { EPI_UP = 0, EPI_DOWN = 1, EPI_LM = 2 };

struct EpiArgs {
  float* out = nullptr;       // act (UP) / h (DOWN) / logits (LM), row stride ldo
  int ldo = 0;
  int N = 0;                  // valid columns
  // UP: 1 / rms from per-tile sums of squares of the block input
  const float* ss_in = nullptr;
  int ss_ld = 0, ss_n = 0;
  float inv_d = 0.f, eps = 0.f;
  // DOWN: next block's normalised input and its sums of squares
  float* xg = nullptr;
  const float* gain_next = nullptr;   // null: last block
  float* ss_out = nullptr;
  // LM: per-tile softmax / argmax statistics of p and of q
  float* pst = nullptr;       // [rows][G][2]
  int* pidx = nullptr;        // [rows][G]   (greedy)
  float* qst = nullptr;       // [B*gamma][G][2]
  const float* q = nullptr;   // [B][gamma][V]
  int G = 0;                  // stats tiles per row
  int G1 = 1, gamma = 0, V = 0;
  int row0 = 0;               // global index of this launch's first row
  int tmode = 0;              // 0 greedy, 1 T == 1, 2 general T
  float invT = 1.f;
};

struct GemmArgs {
  const float* X = nullptr;   // [M][ldx] fp32, columns >= K are zero
  int ldx = 0, M = 0, K = 0;
  const void* W = nullptr;
  int Np = 0, KS = 0, G = 0;  // KS = Kp / 32, G = Np / 64
  int S = 1, kps = 0;         // splits, k-steps per split
  float* part = nullptr;      // [S][M][Np]
  int* cnt = nullptr;         // [G], zero on entry, left zero on exit
  EpiArgs e;
};

// Launch plan of one GEMM (chosen on the host).
enum GemmPath { PATH_FMA_F32 = 0, PATH_FMA_BF16 = 1, PATH_MFMA = 2 };

void choose_split(int path, int M, int KS, int G, int& S, int& kps);
hipError_t launch_gemm(int path, int epi, const GemmArgs& a, hipStream_t st);
size_t gemm_part_floats(int path, int M, const Mat& m);

// Sampling-side launchers (sample.hip).
struct SampleArgs {
  int B = 0, gamma = 0, V = 0, G = 0;
  int M = 0;                  // B * (gamma + 1)
  const float* logits = nullptr; int ldl = 0;
  const float* q = nullptr;
  const int* draft = nullptr;
  float T = 1.f, invT = 1.f, top_p = 1.f;
  int tmode = 0;
  uint64_t seed = 0;
  int* n_acc = nullptr; int* emitted = nullptr;
  float* pst = nullptr; int* pidx = nullptr; float* qst = nullptr;
  float* rowinfo = nullptr;   // [M + B*gamma][8]
  int* dec = nullptr;         // [B][4]
  double* csum = nullptr;     // [B][nch][2]
  int nch = 0;
  float* p_out = nullptr; float* q_out = nullptr;   // debug dumps
};

hipError_t launch_prep(float* h, float* xg, float* ss, int ss_ld, const float* hidden,
                       const float* gain0, int M, int d, int ld, int* cnt, int ncnt,
                       hipStream_t st);
hipError_t launch_tile_stats(const SampleArgs& a, hipStream_t st);
hipError_t launch_sampling(const SampleArgs& a, hipStream_t st);
hipError_t launch_dump_probs(const SampleArgs& a, hipStream_t st);

// Weight conversion launchers (pack.hip).
hipError_t launch_pack_mfma(const void* src, int src_dtype, int K, int N, void* dst, int Kp,
                            int Np, hipStream_t st);
hipError_t launch_copy_rowmajor(const void* src, int src_dtype, int K, int N, void* dst,
                                int dst_dtype, int Kp, int Np, hipStream_t st);
hipError_t launch_vec_to_f32(const void* src, int src_dtype, int n, float* dst, hipStream_t st);

constexpr int kResampleChunk = 4096;   // elements per resample chunk

}  // namespace sv
