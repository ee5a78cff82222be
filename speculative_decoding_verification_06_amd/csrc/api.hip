// C ABI of the verification step: argument checks, workspace layout, weight
// registration and the launch sequence (target pass, then the rule).

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <mutex>
#include <new>
#include <vector>

#include "common.h"
#include "internal.h"
#include "specverify.h"
#include "specverify_diag.h"

using namespace sv;

// Scratch of the allocation-free entry point: one array per GPU, holding
// the pass's workspace for callers that cannot allocate.  In host code the
// name `scratch` is a host-side stand-in, never a device address: its device
// address is taken once per device with hipGetSymbolAddress and kept in
// g_scratch; kernels receive that pointer like any workspace.
constexpr size_t kScratchBytes = SPEC_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this device's scratch (the current device must be
// `dev`); nullptr when the lookup fails.
void* scratch_address(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}
}  // namespace

struct spec_weights {
  int d = 0, ffn = 0, n_blocks = 0, V = 0, wdtype = 0;
  float eps = 0.f;
  uint32_t flags = 0;
  int mfma_min_rows = 1;
  int device = 0;
  void* scratch = nullptr;          // this device's scratch (spec_verify_noalloc)
  std::vector<Mat> up, down;
  Mat lm;
  std::vector<float*> gain;
  // optional GEMM timing (spec_profile_*)
  bool prof = false;
  std::vector<hipEvent_t> ev;       // pairs: [2i] before, [2i+1] after launch i
  std::vector<int64_t> ev_bytes;    // algorithmic weight bytes of launch i
  size_t ev_used = 0;               // launches recorded
};

namespace {

constexpr int kDefaultMfmaMinRows = 1;
constexpr int kMaxGamma = 4096;
constexpr int kMaxRowsMfma = 224;
constexpr int kMaxRowsFma = 160;   // LDS: 160 result rows and 8 waves' sums within 64 KiB

inline int roundup(int x, int m) { return (x + m - 1) / m * m; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Layout {
  int M = 0, ldd = 0, ldf = 0, Vs = 0, G = 0, Gu = 0, nch = 0;
  int ksd = 0, ksf = 0;       // k-steps of the d- and ffn-wide split inputs
  size_t h = 0, xg = 0, ss = 0, act = 0, logits = 0, pst = 0, pidx = 0, qst = 0, rowinfo = 0,
         dec = 0, csum = 0, xsd = 0, xsf = 0, part = 0, rms = 0, total = 0;
};

int gemm_path(const spec_weights* w, int M) {
  if (w->wdtype == SPEC_F32) return PATH_FMA_F32;
  const bool have_rm = w->lm.rowmajor != nullptr;
  return (M >= w->mfma_min_rows || !have_rm) ? PATH_MFMA : PATH_FMA_BF16;
}

// Whether a pass of M rows carries its activations as two bf16 terms, unless
// the weights were registered with SPEC_FLAG_EXACT_SPLIT: every pass the
// wide GEMM serves, whose k-loop chain of activation loads, LDS reads and
// matrix operations per k-step then shrinks by a third (measured 10.6% of a
// 72-row top-p pass and 14-21% of B = 1 passes of 65 to 97 rows), and the
// stacked passes of 6 to 8 rows, whose eight rows of two terms fit one
// fragment where five rows of three do not.  Stacked passes of up to 5 rows
// keep three exact terms, which cost no extra matrix operation there.  Every
// producer of the pass splits alike.
bool two_term(const spec_weights* w, int M, int path) {
  return !(w->flags & SPEC_FLAG_EXACT_SPLIT) && path == PATH_MFMA &&
         (wide_rows(M) || (M >= 6 && M <= kStackRows2));
}

// Statistics units per logits row: one per LM-head work group (nt tiles of
// 16 columns; the vector-FMA path covers 4 tiles per work group).
int lm_units(const spec_weights* w, int M) {
  const int path = gemm_path(w, M);
  const bool wide = path == PATH_MFMA && wide_rows(M);   // epilogue in 64-column blocks
  const int nt = (path == PATH_MFMA && !wide) ? w->lm.nt : kGroupCols / kSub;
  return w->lm.Np / kSub / nt;
}

int max_rows(int path) { return path == PATH_MFMA ? kMaxRowsMfma : kMaxRowsFma; }

// fp32 partial-sum buffer of the wide GEMMs: the largest S x rows x Np over
// the pass's GEMMs (rows of one chunk).
size_t wide_part_bytes(const spec_weights* w, int M) {
  const int path = gemm_path(w, M);
  if (path != PATH_MFMA || !wide_rows(M)) return 0;
  const int rows = M;
  size_t best = 0;
  auto one = [&](const Mat& m) {
    const WidePlan p = plan_wide(rows, m, two_term(w, M, path));
    best = std::max(best, (size_t)p.S * rows * m.Np * sizeof(float));
  };
  for (const Mat& m : w->up) one(m);
  for (const Mat& m : w->down) one(m);
  one(w->lm);
  return best;
}

// Sampling-side buffers, shared by both entry points.
// G statistics units per row, stored at an even stride Gs so rows load in
// 16-byte pairs.
void layout_sampling(Layout& L, int B, int gamma, int V, int G, size_t& off) {
  L.Gu = G;
  L.G = (G + 1) & ~1;
  L.nch = (V + kResampleChunk - 1) / kResampleChunk;
  const size_t qrows = (size_t)B * gamma;
  L.pst = off; off = align256(off + sizeof(float) * 2 * (size_t)L.M * L.G);
  L.pidx = off; off = align256(off + sizeof(int) * (size_t)L.M * L.G);
  L.qst = off; off = align256(off + sizeof(float) * 2 * qrows * L.G);
  L.rowinfo = off; off = align256(off + sizeof(float) * 8 * ((size_t)L.M + qrows));
  L.dec = off; off = align256(off + sizeof(int) * 4 * (size_t)B);
  L.csum = off; off = align256(off + sizeof(double) * 2 * (size_t)B * L.nch);
}

Layout make_layout(const spec_weights* w, int B, int gamma) {
  Layout L;
  L.M = B * (gamma + 1);
  L.ldd = roundup(w->d, kGroupCols);
  L.ldf = roundup(w->ffn, kGroupCols);
  L.Vs = roundup(w->V, kGroupCols);
  size_t off = 0;
  const size_t M = L.M;
  L.h = off; off = align256(off + sizeof(float) * M * L.ldd);
  L.xg = off; off = align256(off + sizeof(float) * M * L.ldd);
  L.ss = off; off = align256(off + sizeof(float) * M * (L.ldd / kSub));
  L.act = off; off = align256(off + sizeof(float) * M * L.ldf);
  L.logits = off; off = align256(off + sizeof(float) * M * L.Vs);
  if (w->wdtype == SPEC_BF16) {
    L.ksd = roundup(w->d, kKStep) / kKStep;
    L.ksf = roundup(w->ffn, kKStep) / kKStep;
    L.xsd = off; off = align256(off + xs_bytes(L.M, L.ksd));
    L.xsf = off; off = align256(off + xs_bytes(L.M, L.ksf));
    L.part = off; off = align256(off + wide_part_bytes(w, L.M));
    L.rms = off; off = align256(off + sizeof(float) * M);
  }
  layout_sampling(L, B, gamma, w->V, lm_units(w, L.M), off);
  L.total = off;
  return L;
}

template <typename T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

bool bad_scalars(float T, float top_p) {
  if (!std::isfinite(T) || T < 0.f) return true;
  if (T > 0.f && !(top_p > 0.f && top_p <= 1.f)) return true;
  return false;
}

int tmode_of(float T) { return T == 0.f ? 0 : (T == 1.f ? 1 : 2); }

void free_weights(spec_weights* w) {
  if (!w) return;
  auto fm = [](Mat& m) {
    if (m.rowmajor) (void)hipFree(m.rowmajor);
    if (m.mfma) (void)hipFree(m.mfma);
    m.rowmajor = m.mfma = nullptr;
  };
  for (auto& m : w->up) fm(m);
  for (auto& m : w->down) fm(m);
  fm(w->lm);
  for (float* g : w->gain)
    if (g) (void)hipFree(g);
  for (hipEvent_t e : w->ev) (void)hipEventDestroy(e);
  delete w;
}

spec_status register_matrix(spec_weights* w, const void* src, int K, int N, bool keep_rm,
                            Mat& m, hipStream_t st) {
  m.K = K; m.N = N; m.Kp = roundup(K, kKStep); m.Np = roundup(N, kGroupCols);
  const size_t elems = (size_t)m.Kp * m.Np;
  if (w->wdtype == SPEC_F32) {
    if (hipMalloc(&m.rowmajor, elems * sizeof(float)) != hipSuccess) { m.rowmajor = nullptr; return SPEC_ENOMEM; }
    if (launch_copy_rowmajor(src, 0, K, N, m.rowmajor, 0, m.Kp, m.Np, st) != hipSuccess) return SPEC_EHIP;
    return SPEC_OK;
  }
  m.nt = mfma_block_tiles(m.Np);
  if (hipMalloc(&m.mfma, elems * sizeof(uint16_t)) != hipSuccess) { m.mfma = nullptr; return SPEC_ENOMEM; }
  if (launch_pack_mfma(src, 1, K, N, m.mfma, m.Kp, m.Np, m.nt, st) != hipSuccess) return SPEC_EHIP;
  if (keep_rm) {
    if (hipMalloc(&m.rowmajor, elems * sizeof(uint16_t)) != hipSuccess) { m.rowmajor = nullptr; return SPEC_ENOMEM; }
    if (launch_copy_rowmajor(src, 1, K, N, m.rowmajor, 1, m.Kp, m.Np, st) != hipSuccess) return SPEC_EHIP;
  }
  return SPEC_OK;
}

const void* mat_ptr(const Mat& m, int path) { return path == PATH_MFMA ? m.mfma : m.rowmajor; }


// Events for timed launch idx (created on first use).
hipError_t prof_events(spec_weights* w, size_t idx, hipEvent_t& e0, hipEvent_t& e1) {
  while (w->ev.size() < 2 * (idx + 1)) {
    hipEvent_t e;
    const hipError_t err = hipEventCreate(&e);
    if (err != hipSuccess) return err;
    w->ev.push_back(e);
  }
  e0 = w->ev[2 * idx];
  e1 = w->ev[2 * idx + 1];
  return hipSuccess;
}

// One GEMM over all M rows, in row chunks the kernels can hold.  Row chunks
// start on 16-row tiles (the chunk sizes are multiples of 16), so a
// chunk's split fragments begin at tile m0 / 16.  With timing on, every
// launch carries a pair of events and its algorithmic weight bytes.
hipError_t run_gemm(spec_weights* w, bool prof, int path, const Mat& W, const float* X,
                    const uint16_t* XS, int ldx, int M, EpiArgs e, float* part, hipStream_t st) {
  const bool two = two_term(w, M, path);
  const int chunk = max_rows(path);
  // the packing and the kernel follow the whole pass's row count (stacked
  // and wide passes are one chunk)
  const bool stack = path == PATH_MFMA && xs_stacked(M);
  const bool wide = path == PATH_MFMA && wide_rows(M);
  static_assert(kMaxRowsMfma % 16 == 0, "MFMA row chunks must start on row tiles");
  for (int m0 = 0; m0 < M; m0 += chunk) {
    GemmArgs a;
    a.X = X + (size_t)m0 * ldx;
    a.XS = XS ? XS + (size_t)(m0 / 16) * (W.Kp / kKStep + 1) * 3 * 512 : nullptr;
    a.ldx = ldx;
    a.M = std::min(chunk, M - m0);
    a.K = W.K;
    a.W = mat_ptr(W, path);
    a.Np = W.Np;
    a.KS = W.Kp / kKStep;
    a.e = e;
    a.e.out = e.out ? e.out + (size_t)m0 * e.ldo : nullptr;
    if (e.kind == EPI_UP) a.e.ss_in = e.ss_in + (size_t)m0 * e.ss_ld;
    if (e.kind == EPI_DOWN) {
      a.e.xg = e.xg + (size_t)m0 * e.ldo;
      a.e.ss_out = e.ss_out + (size_t)m0 * e.ss_ld;
    }
    if (e.xs) a.e.xs = e.xs + (size_t)(m0 / 16) * (e.xs_ks + 1) * 3 * 512;
    a.e.xs_stack = stack;
    a.e.xs_two = two;
    a.e.row0 = m0;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (prof) {
      const hipError_t err = prof_events(w, w->ev_used, e0, e1);
      if (err != hipSuccess) return err;
    }
    hipError_t err;
    if (wide) {
      const WidePlan wp = plan_wide(a.M, W, two);
      WideArgs wa;
      wa.XS = a.XS; wa.W = W.mfma; wa.M = a.M; wa.MT = wp.MT; wa.KS = a.KS;
      wa.nt = W.nt; wa.tiles = W.Np / kSub; wa.ks_slice = wp.ks_slice; wa.S = wp.S;
      wa.P = part; wa.ldp = W.Np; wa.slice_stride = (size_t)a.M * W.Np;
      err = launch_wide(wp, wa, a.e, st, e0, e1);
    } else {
      err = launch_gemm(plan_gemm(path, a.M, W, stack, two), a, st, e0, e1);
    }
    if (err != hipSuccess) return err;
    if (prof) {
      w->ev_bytes.resize(w->ev_used + 1);
      w->ev_bytes[w->ev_used] = (int64_t)W.K * W.N * (w->wdtype == SPEC_F32 ? 4 : 2);
      ++w->ev_used;
    }
  }
  return hipSuccess;
}

spec_status check_device(const spec_weights* w) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SPEC_EHIP;
  return dev == w->device ? SPEC_OK : SPEC_EINVAL;
}

// Draft tree of a greedy tree verification (spec_verify_tree_greedy).
struct TreeArgs {
  const int32_t* parent = nullptr;   // [B][n]
  const int32_t* tokens = nullptr;   // [B][n]
  int32_t* path = nullptr;           // [B][n] or null
};

spec_status verify_impl(spec_weights_t w, int32_t B, int32_t gamma, const float* hidden,
                        const int32_t* draft, const float* q, float T, float top_p,
                        uint64_t seed, int32_t* n_acc, int32_t* emitted, void* ws,
                        size_t ws_bytes, void* stream, float* logits_out, float* p_out,
                        float* q_out, bool noalloc = false, const TreeArgs* tree = nullptr) {
  if (!w || B < 1 || gamma < 0 || gamma > kMaxGamma || !hidden || !n_acc || !emitted)
    return SPEC_EINVAL;
  if (tree && gamma > 0 && (!tree->parent || !tree->tokens)) return SPEC_EINVAL;
  if (!tree && gamma > 0 && !draft) return SPEC_EINVAL;
  if (bad_scalars(T, top_p)) return SPEC_EINVAL;
  if (T > 0.f && gamma > 0 && !q) return SPEC_EINVAL;
  if ((size_t)B * (gamma + 1) > (size_t)INT32_MAX / 2) return SPEC_EINVAL;
  const Layout L = make_layout(w, B, gamma);
  if (noalloc) {
    if (L.total > kScratchBytes) return SPEC_ESCRATCH;
    ws = w->scratch;
    ws_bytes = kScratchBytes;
    if (!ws) return SPEC_EHIP;
  }
  if (!ws || ws_bytes < L.total || (reinterpret_cast<uintptr_t>(ws) & 255)) return SPEC_EWORKSPACE;
  if (spec_status s = check_device(w); s != SPEC_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  // timing events are created on demand: never on the allocation-free path
  const bool prof = w->prof && !noalloc;

  const int M = L.M, path = gemm_path(w, M);
  float* h = at<float>(ws, L.h);
  float* xg = at<float>(ws, L.xg);
  float* ss = at<float>(ws, L.ss);
  float* act = at<float>(ws, L.act);
  float* logits = at<float>(ws, L.logits);
  float* part = L.part ? at<float>(ws, L.part) : nullptr;
  // per-row 1 / rms for the wide GEMM's UP epilogue (computed once per pass)
  float* rms = path == PATH_MFMA && wide_rows(M) ? at<float>(ws, L.rms) : nullptr;
  const int ss_ld = L.ldd / kSub;
  const int tmode = tmode_of(T);
  // split activations, for the MFMA path only
  uint16_t* xsd = path == PATH_MFMA ? at<uint16_t>(ws, L.xsd) : nullptr;
  uint16_t* xsf = path == PATH_MFMA ? at<uint16_t>(ws, L.xsf) : nullptr;

  hipError_t err = launch_prep(h, xg, ss, ss_ld, hidden, w->n_blocks ? w->gain[0] : nullptr, M,
                               w->d, L.ldd, xsd, L.ksd, xsf, L.ksf, two_term(w, M, path), st);
  for (int l = 0; l < w->n_blocks && err == hipSuccess; ++l) {
    EpiArgs up;
    up.kind = EPI_UP;
    up.out = act; up.ldo = L.ldf; up.N = w->ffn;
    up.ss_in = ss; up.ss_ld = ss_ld; up.ss_n = ss_ld;
    up.inv_d = 1.0f / (float)w->d; up.eps = w->eps;
    up.rms = rms;
    up.xs = xsf; up.xs_ks = L.ksf;
    err = run_gemm(w, prof, path, w->up[l], xg, xsd, L.ldd, M, up, part, st);
    if (err != hipSuccess) break;
    EpiArgs dn;
    dn.kind = EPI_DOWN;
    dn.out = h; dn.ldo = L.ldd; dn.N = w->d;
    dn.xg = xg; dn.gain_next = l + 1 < w->n_blocks ? w->gain[l + 1] : nullptr;
    dn.ss_out = ss; dn.ss_ld = ss_ld;
    dn.xs = xsd; dn.xs_ks = L.ksd;
    err = run_gemm(w, prof, path, w->down[l], act, xsf, L.ldf, M, dn, part, st);
  }
  if (err == hipSuccess) {
    EpiArgs lm;
    lm.kind = EPI_LM;
    // greedy passes read only the argmax statistics: no logits unless asked for
    lm.out = tmode == 0 && !logits_out ? nullptr : logits; lm.ldo = L.Vs; lm.N = w->V;
    lm.pst = at<float>(ws, L.pst); lm.pidx = at<int>(ws, L.pidx); lm.qst = at<float>(ws, L.qst);
    lm.q = q; lm.G = L.G; lm.G1 = gamma + 1; lm.gamma = gamma; lm.V = w->V;
    lm.tmode = tmode; lm.invT = tmode ? 1.0f / T : 1.0f;
    err = run_gemm(w, prof, path, w->lm, h, xsd, L.ldd, M, lm, part, st);
  }
  SampleArgs sa;
  if (err == hipSuccess) {
    sa.B = B; sa.gamma = gamma; sa.V = w->V; sa.G = L.G; sa.Gu = L.Gu; sa.M = M;
    sa.logits = logits; sa.ldl = L.Vs; sa.q = q; sa.draft = draft;
    sa.T = T; sa.invT = tmode ? 1.0f / T : 1.0f; sa.top_p = top_p; sa.tmode = tmode; sa.seed = seed;
    sa.n_acc = n_acc; sa.emitted = emitted;
    sa.pst = at<float>(ws, L.pst); sa.pidx = at<int>(ws, L.pidx); sa.qst = at<float>(ws, L.qst);
    sa.rowinfo = at<float>(ws, L.rowinfo); sa.dec = at<int>(ws, L.dec);
    sa.csum = at<double>(ws, L.csum); sa.nch = L.nch;
    err = tree ? launch_tree_walk(sa, tree->parent, tree->tokens, tree->path, st)
               : launch_sampling(sa, st);
  }
  if (err == hipSuccess && (p_out || q_out)) {
    sa.p_out = p_out; sa.q_out = q_out;
    err = launch_dump_probs(sa, st);
  }
  if (err == hipSuccess && logits_out)
    err = hipMemcpy2DAsync(logits_out, sizeof(float) * w->V, logits, sizeof(float) * L.Vs,
                           sizeof(float) * w->V, M, hipMemcpyDeviceToDevice, st);
  return err == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

// ---------------------------------------------------------------- access check
// Host-side model of every global and LDS access the kernels of one pass
// make, at the extremes of their index ranges (the block, wave, lane and
// k-step that reach the lowest and highest element of each buffer), for the
// launch plans verify_impl would choose.  The address formulas are the
// kernels' own (xs_index is shared with them; the rest restate gemm.hip's
// k_gemm_mfma, k_gemm_wide, k_epi_wide, k_epi_wide8, k_gemm_fma, run_epilogue and
// sample.hip's k_prep line for line).  Nothing is launched.
struct AccessCheck {
  char* msg = nullptr;
  size_t msg_len = 0;
  int64_t checks = 0;
  bool ok = true;
  void range(const char* what, const char* buf, int64_t lo, int64_t hi, int64_t cap) {
    ++checks;
    if (lo >= 0 && hi < cap) return;
    if (ok && msg && msg_len)
      snprintf(msg, msg_len, "%s: %s elements [%lld, %lld] outside [0, %lld)", what, buf,
               (long long)lo, (long long)hi, (long long)cap);
    ok = false;
  }
};

// Buffer capacities of a pass, in the unit each kernel indexes them with.
struct PassBufs {
  int64_t h, xg, ss, act, logits, pst, pidx, qst, xsd, xsf, part, rms;
};

PassBufs pass_bufs(const spec_weights* w, const Layout& L, int B, int gamma, int shrink) {
  PassBufs c;
  const int64_t M = L.M;
  c.h = c.xg = M * L.ldd;
  c.ss = M * (L.ldd / kSub);
  c.act = M * L.ldf;
  c.logits = M * L.Vs;
  c.pst = 2 * M * L.G;
  c.pidx = M * L.G;
  c.qst = 2 * (int64_t)B * gamma * L.G;
  c.xsd = L.ksd ? (int64_t)xs_bytes(L.M, L.ksd) / 2 : 0;   // bf16 elements
  c.xsf = L.ksf ? (int64_t)xs_bytes(L.M, L.ksf) / 2 : 0;
  c.part = (int64_t)wide_part_bytes(w, L.M) / 4;
  c.rms = M;
  if (shrink > 0) {
    // a planted inconsistency: every buffer `shrink` bytes short
    for (int64_t* x : {&c.h, &c.xg, &c.ss, &c.act, &c.logits, &c.pst, &c.pidx, &c.qst, &c.part, &c.rms})
      *x -= (shrink + 3) / 4;
    c.xsd -= (shrink + 1) / 2;
    c.xsf -= (shrink + 1) / 2;
  }
  return c;
}

// Split-activation stores of an epilogue or of k_prep: pass rows [row0,
// row0 + rows), columns below cols and below 32 ks.  A chunk's kernels add
// the chunk's first row tile to the buffer pointer and index with local
// rows, which for the plain packing (16-row tiles, chunks on tile bounds)
// is xs_index of the pass row.
void check_xs_store(AccessCheck& C, const char* what, const char* buf, int64_t cap, int row0,
                    int rows, int cols, int ks, bool stacked, bool two) {
  const int ncol = std::min(cols, kKStep * ks);
  if (rows <= 0 || ncol <= 0) return;
  int64_t lo = INT64_MAX, hi = -1;
  const int st = xs_term_step(stacked, two), last_term = two ? 1 : 2;
  const int last = (ncol - 1) / kKStep;   // columns of the first and last k-step
  for (int r = row0; r < row0 + rows; ++r)
    for (int s = 0; s <= last; s += std::max(1, last))
      for (int j = 0; j < kKStep; ++j) {
        const int col = s * kKStep + j;
        if (col >= ncol) break;
        const int64_t i = (int64_t)xs_index(r, col, ks, stacked, two);
        lo = std::min(lo, i);
        hi = std::max(hi, i + last_term * st);
      }
  C.range(what, buf, lo, hi, cap);
}

// Epilogue accesses for rows [row0, row0 + rows) of the pass and 16-column
// tiles [t0, t1) of the GEMM's output.
struct EpiCheck {
  int kind, N, Np, ldo, nt;                // nt: tiles of one statistics unit
  bool to_xs, stacked, two;
  int xs_ks;
  const char* xs_name;
  int64_t xs_cap;                          // next GEMM's split buffer (bf16 elements)
  bool wide_rms;
  int B, gamma, V, G, M_total;
};

void check_epilogue(AccessCheck& C, const char* what, const EpiCheck& e, const PassBufs& c,
                    const Layout& L, int row0, int rows, int t0, int t1) {
  if (rows <= 0 || t1 <= t0) return;
  const int nlast = t1 * kSub - 1;         // highest column a live item touches
  const int64_t r_lo = row0, r_hi = row0 + rows - 1;
  const int ss_ld = L.ldd / kSub;
  if (e.kind == EPI_UP) {
    if (e.wide_rms) C.range(what, "rms", r_lo, r_hi, c.rms);
    else C.range(what, "ss (sums of squares)", r_lo * ss_ld, r_hi * ss_ld + ss_ld - 1, c.ss);
    if (!e.to_xs) C.range(what, "act", r_lo * e.ldo + t0 * kSub, r_hi * e.ldo + nlast, c.act);
  } else if (e.kind == EPI_DOWN) {
    C.range(what, "h", r_lo * e.ldo + t0 * kSub, r_hi * e.ldo + nlast, c.h);
    if (!e.to_xs) C.range(what, "xg", r_lo * e.ldo + t0 * kSub, r_hi * e.ldo + nlast, c.xg);
    C.range(what, "ss (sums of squares)", r_lo * ss_ld + t0, r_hi * ss_ld + t1 - 1, c.ss);
  } else {
    const int nv = std::min(nlast, e.N - 1);
    C.range(what, "logits", r_lo * e.ldo + t0 * kSub, r_hi * e.ldo + nv, c.logits);
    const int u0 = t0 / e.nt, u1 = (t1 - 1) / e.nt;
    C.range(what, "pst", 2 * (r_lo * e.G + u0), 2 * (r_hi * e.G + u1) + 1, c.pst);
    C.range(what, "pidx", r_lo * e.G + u0, r_hi * e.G + u1, c.pidx);
    // draft rows among them: b * gamma + i for rows b (gamma + 1) + i, i < gamma
    int64_t q_lo = INT64_MAX, q_hi = -1;
    for (int64_t g = r_lo; g <= r_hi; ++g) {
      const int64_t b = g / (e.gamma + 1), i = g - b * (e.gamma + 1);
      if (i < e.gamma) { q_lo = std::min(q_lo, b * e.gamma + i); q_hi = std::max(q_hi, b * e.gamma + i); }
    }
    if (q_hi >= 0) C.range(what, "qst", 2 * (q_lo * e.G + u0), 2 * (q_hi * e.G + u1) + 1, c.qst);
  }
  if (e.to_xs) check_xs_store(C, what, e.xs_name, e.xs_cap, row0, rows, t1 * kSub, e.xs_ks, e.stacked, e.two);
}

void check_mfma(AccessCheck& C, const char* what, const GemmPlan& p, const Mat& W, int M,
                const char* xs_name, int64_t xs_cap, int64_t xs_off_units, const EpiCheck& e,
                const PassBufs& c, const Layout& L, int row0) {
  const int KS = W.Kp / kKStep, NT = p.nt;
  const int FPT = p.stack ? 1 : 3, RPT = p.stack ? xs_stack_rows(p.two) : 16;
  const int TERMS = p.stack ? (p.two ? 2 : 3) : 1;
  const int MT = (M + RPT - 1) / RPT, MG = p.mg, KG = p.kg, nwaves = MG * KG;
  const int64_t wcap = (int64_t)W.Kp * W.Np / 8;     // bf16x8 fragments
  if ((int64_t)p.blocks * NT * kSub != W.Np) { C.range(what, "column blocks", 0, p.blocks * NT * kSub, W.Np + 1); }
  for (int bx : {0, p.blocks - 1})
    for (int wave = 0; wave < nwaves; ++wave) {
      const int mg = wave % MG, kg = wave / MG, mt0 = mg * p.mtw;
      if (!(mt0 < MT) || kg >= KS) continue;
      const int n = (KS - kg + KG - 1) / KG, klast = kg + (n - 1) * KG;
      const int64_t wg = (int64_t)bx * KS * NT * 64;
      C.range(what, "weights", wg + (int64_t)kg * NT * 64, wg + 63 + (int64_t)klast * NT * 64 + (NT - 1) * 64, wcap);
      for (int i = 0; i < p.mtw; ++i) {
        const int mt = std::min(mt0 + i, MT - 1);
        const int rows = std::min(RPT, M - mt * RPT);
        for (int lane = 0; lane < 64; lane += 63) {
          const int ar = lane & 15;
          int al;
          if (p.stack) {
            const int pp = std::min(ar / RPT, TERMS - 1);
            al = (lane & 48) + pp * RPT + std::min(ar - pp * RPT, rows - 1);
          } else {
            al = (lane & 48) + std::min(ar, rows - 1);
          }
          const int64_t base = xs_off_units + (int64_t)mt * (KS + 1) * FPT * 64 + al;
          C.range(what, xs_name, base + (int64_t)kg * FPT * 64, base + (int64_t)KS * FPT * 64 + (FPT - 1) * 64, xs_cap);
        }
      }
    }
  const int ldr = NT * kSub + 1;
  const int64_t lds = (int64_t)p.lds / 4;
  C.range(what, "LDS k-group tiles", 0, ((((int64_t)KG - 1) * M + M - 1) * TERMS + TERMS - 1) * ldr + NT * kSub - 1, lds);
  if (p.stack) C.range(what, "LDS summed tile", 0, (int64_t)KG * M * TERMS * ldr + (int64_t)(M - 1) * ldr + NT * kSub - 1, lds);
  check_epilogue(C, what, e, c, L, row0, M, 0, NT);
  check_epilogue(C, what, e, c, L, row0, M, (p.blocks - 1) * NT, p.blocks * NT);
}

void check_wide(AccessCheck& C, const char* what, const WidePlan& p, const Mat& W, int M,
                const char* xs_name, int64_t xs_cap, const EpiCheck& e, const PassBufs& c,
                const Layout& L) {
  const int KS = W.Kp / kKStep, MT = p.MT, tiles = W.Np / kSub;
  const int threads = 64 * p.mg * p.cg;
  const int fr = p.terms * 64;   // chunks of a row tile's k-step the GEMM reads
  const int cpt = (p.mtw * p.mg * fr + threads - 1) / threads;
  const int64_t nfrp = (int64_t)cpt * threads, nfr = (int64_t)MT * fr;
  const int64_t wcap = (int64_t)W.Kp * W.Np / 8;
  C.range(what, "LDS activation tiles", 0, 2 * nfrp - 1, (int64_t)p.lds / 16);
  for (int by = 0; by < p.S; ++by) {
    const int s0 = by * p.ks_slice, s1 = std::min(KS, s0 + p.ks_slice);
    if (s1 <= s0) continue;
    for (int tid = 0; tid < threads; tid += threads - 1)
      for (int i = 0; i < cpt; ++i) {
        const int64_t cc = std::min<int64_t>(tid + (int64_t)i * threads, nfr - 1);
        const int64_t mt = cc / fr, rem = cc - mt * fr;
        const int64_t base = mt * (KS + 1) * 192 + rem;
        C.range(what, xs_name, base + (int64_t)s0 * 192, base + (int64_t)KS * 192, xs_cap);
      }
    for (int bx : {0, p.colblocks - 1})
      for (int cg = 0; cg < p.cg; ++cg)
        for (int t = 0; t < p.ntc; ++t) {
          const int tile = bx * (p.ntc * p.cg) + cg * p.ntc + t;
          const int tt = std::min(tile, tiles - 1);
          const int b = tt / W.nt, tp = tt - b * W.nt;
          const int64_t wp = ((int64_t)b * KS * W.nt + tp) * 64;
          C.range(what, "weights", wp + (int64_t)s0 * W.nt * 64, wp + 63 + (int64_t)(s1 - 1) * W.nt * 64, wcap);
        }
  }
  const bool fuse_lm = p.S == 1 && e.kind == EPI_LM;
  if (fuse_lm) {
    if (p.ntc == 2) {
      const int64_t R = (int64_t)p.mg * p.mtw * 16;
      C.range(what, "LDS half-unit statistics", 0, (int64_t)p.cg * R * 16 - 1, (int64_t)p.lds);
    }
    check_epilogue(C, what, e, c, L, 0, M, 0, 4);
    check_epilogue(C, what, e, c, L, 0, M, tiles - 4, tiles);
    return;
  }
  // partial sums P[slice][row][col], then the slice-sum epilogue per 16 rows
  // (k_epi_wide8: 128 columns for UP and DOWN; k_epi_wide: 4 tiles for LM)
  const int64_t ss = (int64_t)M * W.Np;
  C.range(what, "partial sums (write)", 0, (int64_t)(p.S - 1) * ss + (int64_t)(M - 1) * W.Np + (tiles - 1) * kSub + 15, c.part);
  for (int by = 0; by * 16 < M; by += std::max(1, ((M + 15) / 16) - 1)) {
    const int m0 = by * 16, mb = std::min(16, M - m0);
    const int64_t c0 = tiles - 4;
    C.range(what, "partial sums (read)", (int64_t)m0 * W.Np,
            (int64_t)(m0 + mb - 1) * W.Np + c0 * kSub + 63 + (int64_t)(p.S - 1) * ss, c.part);
    check_epilogue(C, what, e, c, L, m0, mb, 0, 4);
    check_epilogue(C, what, e, c, L, m0, mb, tiles - 4, tiles);
    if (by == (M + 15) / 16 - 1) break;
  }
}

void check_fma(AccessCheck& C, const char* what, const GemmPlan& p, const Mat& W, int M, int ldx,
               int64_t x_cap, const char* x_name, int64_t x_off, const EpiCheck& e,
               const PassBufs& c, const Layout& L, int row0) {
  const int Kp = W.Kp;
  C.range(what, x_name, x_off, x_off + (int64_t)(M - 1) * ldx + Kp - 1, x_cap);
  C.range(what, "weights (row-major)", 0, (int64_t)(p.blocks - 1) * kGroupCols + 63 + (int64_t)(Kp - 1) * W.Np,
          (int64_t)Kp * W.Np);
  C.range(what, "LDS", 0, (int64_t)M * (kGroupCols + 1) + kFmaWaves * 8 * (kGroupCols + 1) - 1,
          (int64_t)p.lds / 4);
  check_epilogue(C, what, e, c, L, row0, M, 0, 4);
  check_epilogue(C, what, e, c, L, row0, M, (p.blocks - 1) * 4, p.blocks * 4);
}

spec_status access_check_pass(const spec_weights* w, int B, int gamma, int shrink, AccessCheck& C) {
  const Layout L = make_layout(w, B, gamma);
  const PassBufs c = pass_bufs(w, L, B, gamma, shrink);
  const int M = L.M, path = gemm_path(w, M);
  const bool stack = path == PATH_MFMA && xs_stacked(M);
  const bool wide = path == PATH_MFMA && wide_rows(M);
  const bool two = two_term(w, M, path);
  // k_prep
  {
    const char* what = "k_prep";
    C.range(what, "h", 0, (int64_t)(M - 1) * L.ldd + L.ldd - 1, c.h);
    C.range(what, "ss (sums of squares)", 0, (int64_t)(M - 1) * (L.ldd / kSub) + L.ldd / kSub - 1, c.ss);
    if (path == PATH_MFMA) {
      check_xs_store(C, what, "xs (d-wide)", c.xsd, 0, M, L.ldd, L.ksd, stack, two);
      // the zero steps of five-row stacked tiles, as k_prep clears them (the
      // eight-row tiles of the two-term packing are a subset)
      const int rpt = stack ? kStackRows : 16, fpt = stack ? 1 : 3;
      const int mtn = (M + rpt - 1) / rpt;
      for (int pass = 0; pass < 2; ++pass) {
        const int ks = pass ? L.ksf : L.ksd;
        const int64_t cap = pass ? c.xsf : c.xsd;
        if (pass && !w->n_blocks) break;
        C.range(what, pass ? "xs zero step (ffn-wide)" : "xs zero step (d-wide)",
                ((int64_t)0 * (ks + 1) + ks) * fpt * 512,
                ((int64_t)(mtn - 1) * (ks + 1) + ks) * fpt * 512 + ((fpt - 1) * 64 + 63) * 8 + 7, cap);
      }
    }
  }
  const int chunk = max_rows(path);
  auto gemm = [&](const char* what, const Mat& W, int kind, bool in_ffn) {
    EpiCheck e;
    e.kind = kind;
    e.N = W.N; e.Np = W.Np;
    e.ldo = kind == EPI_UP ? L.ldf : (kind == EPI_DOWN ? L.ldd : L.Vs);
    e.stacked = stack;
    e.two = two;
    e.to_xs = path == PATH_MFMA && kind != EPI_LM;
    e.xs_ks = kind == EPI_UP ? L.ksf : L.ksd;
    e.xs_name = kind == EPI_UP ? "xs (ffn-wide, next input)" : "xs (d-wide, next input)";
    e.xs_cap = kind == EPI_UP ? c.xsf : c.xsd;
    e.wide_rms = wide && kind == EPI_UP;
    e.B = B; e.gamma = gamma; e.V = w->V; e.G = L.G; e.M_total = M;
    const char* xs_name = in_ffn ? "xs (ffn-wide)" : "xs (d-wide)";
    const int64_t xs_cap = in_ffn ? c.xsf : c.xsd;
    for (int m0 = 0; m0 < M; m0 += chunk) {
      const int Mc = std::min(chunk, M - m0);
      const int64_t xs_off = (int64_t)(m0 / 16) * (W.Kp / kKStep + 1) * 3 * 64;   // fragments
      if (path != PATH_MFMA) {
        const int ldx = in_ffn ? L.ldf : L.ldd;
        const int64_t x_cap = in_ffn ? c.act : (kind == EPI_LM ? c.h : c.xg);
        e.nt = 4;
        check_fma(C, what, plan_gemm(path, Mc, W, false, false), W, Mc, ldx, x_cap,
                  in_ffn ? "act" : (kind == EPI_LM ? "h" : "xg"), (int64_t)m0 * ldx, e, c, L, m0);
      } else if (wide) {
        e.nt = kGroupCols / kSub;
        check_wide(C, what, plan_wide(Mc, W, two), W, Mc, xs_name, xs_cap / 8, e, c, L);
      } else {
        const GemmPlan p = plan_gemm(path, Mc, W, stack, two);
        e.nt = p.nt;
        check_mfma(C, what, p, W, Mc, xs_name, xs_cap / 8, xs_off, e, c, L, m0);
      }
    }
  };
  char name[64];
  for (int l = 0; l < w->n_blocks; ++l) {
    snprintf(name, sizeof name, "up projection, block %d", l);
    gemm(name, w->up[l], EPI_UP, false);
    snprintf(name, sizeof name, "down projection, block %d", l);
    gemm(name, w->down[l], EPI_DOWN, true);
  }
  gemm("LM head", w->lm, EPI_LM, false);
  return C.ok ? SPEC_OK : SPEC_EINVAL;
}

}  // namespace

extern "C" {

const char* spec_status_string(spec_status s) {
  switch (s) {
    case SPEC_OK: return "ok";
    case SPEC_EINVAL: return "invalid argument";
    case SPEC_EDTYPE: return "unsupported weight dtype";
    case SPEC_EWORKSPACE: return "workspace missing, misaligned or too small";
    case SPEC_EHIP: return "HIP runtime error";
    case SPEC_ENOMEM: return "device allocation failed";
    case SPEC_ESCRATCH: return "pass needs more workspace than the allocation-free scratch holds";
  }
  return "unknown status";
}

int32_t spec_default_mfma_min_rows(void) { return kDefaultMfmaMinRows; }

spec_status spec_weights_create(const spec_weights_desc* desc, void* stream, spec_weights_t* out) {
  if (!desc || !out) return SPEC_EINVAL;
  if (desc->wdtype != SPEC_F32 && desc->wdtype != SPEC_BF16) return SPEC_EDTYPE;
  if (desc->d < 1 || desc->ffn < 1 || desc->vocab < 1 || desc->n_blocks < 0) return SPEC_EINVAL;
  if (!std::isfinite(desc->rms_eps) || desc->rms_eps < 0.f || !desc->lm_head) return SPEC_EINVAL;
  if (desc->n_blocks > 0 && (!desc->w_up || !desc->w_down)) return SPEC_EINVAL;
  for (int l = 0; l < desc->n_blocks; ++l) {
    if (!desc->w_up[l] || !desc->w_down[l]) return SPEC_EINVAL;
    if (desc->norm_gain && !desc->norm_gain[l]) return SPEC_EINVAL;
  }
  spec_weights* w = new (std::nothrow) spec_weights;
  if (!w) return SPEC_ENOMEM;
  w->d = desc->d; w->ffn = desc->ffn; w->n_blocks = desc->n_blocks; w->V = desc->vocab;
  w->wdtype = desc->wdtype; w->eps = desc->rms_eps; w->flags = desc->flags;
  w->mfma_min_rows = desc->mfma_min_rows > 0 ? desc->mfma_min_rows : kDefaultMfmaMinRows;
  if (hipGetDevice(&w->device) != hipSuccess) { delete w; return SPEC_EHIP; }
  // set-up of the allocation-free entry point: this device's scratch address
  w->scratch = scratch_address(w->device);
  if (!w->scratch) { delete w; return SPEC_EHIP; }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool keep_rm = w->wdtype == SPEC_BF16 &&
                       ((desc->flags & SPEC_FLAG_KEEP_ROWMAJOR) || w->mfma_min_rows > 1);
  w->up.resize(w->n_blocks);
  w->down.resize(w->n_blocks);
  w->gain.assign(w->n_blocks, nullptr);
  spec_status s = SPEC_OK;
  for (int l = 0; l < w->n_blocks && s == SPEC_OK; ++l) {
    s = register_matrix(w, desc->w_up[l], w->d, w->ffn, keep_rm, w->up[l], st);
    if (s == SPEC_OK) s = register_matrix(w, desc->w_down[l], w->ffn, w->d, keep_rm, w->down[l], st);
    if (s == SPEC_OK) {
      if (hipMalloc(&w->gain[l], sizeof(float) * w->d) != hipSuccess) { w->gain[l] = nullptr; s = SPEC_ENOMEM; }
      else if (launch_vec_to_f32(desc->norm_gain ? desc->norm_gain[l] : nullptr, w->wdtype, w->d,
                                 w->gain[l], st) != hipSuccess) s = SPEC_EHIP;
    }
  }
  if (s == SPEC_OK) s = register_matrix(w, desc->lm_head, w->d, w->V, keep_rm, w->lm, st);
  if (s == SPEC_OK && hipStreamSynchronize(st) != hipSuccess) s = SPEC_EHIP;
  if (s != SPEC_OK) {
    (void)hipStreamSynchronize(st);
    free_weights(w);
    return s;
  }
  *out = w;
  return SPEC_OK;
}

spec_status spec_weights_destroy(spec_weights_t w) {
  if (w) {
    int prev = 0;
    (void)hipGetDevice(&prev);
    (void)hipSetDevice(w->device);
    (void)hipDeviceSynchronize();
    free_weights(w);
    (void)hipSetDevice(prev);
  }
  return SPEC_OK;
}

spec_status spec_profile_enable(spec_weights_t w, int32_t on) {
  if (!w) return SPEC_EINVAL;
  w->prof = on != 0;
  w->ev_used = 0;
  return SPEC_OK;
}

spec_status spec_profile_read(spec_weights_t w, double* gemm_ms, int64_t* launches,
                              int64_t* weight_bytes) {
  if (!w) return SPEC_EINVAL;
  double ms = 0.0;
  int64_t bytes = 0;
  if (w->ev_used) {
    if (hipEventSynchronize(w->ev[2 * w->ev_used - 1]) != hipSuccess) return SPEC_EHIP;
    for (size_t i = 0; i < w->ev_used; ++i) {
      float t = 0.f;
      if (hipEventElapsedTime(&t, w->ev[2 * i], w->ev[2 * i + 1]) != hipSuccess) return SPEC_EHIP;
      ms += t;
      bytes += w->ev_bytes[i];
    }
  }
  if (gemm_ms) *gemm_ms = ms;
  if (launches) *launches = (int64_t)w->ev_used;
  if (weight_bytes) *weight_bytes = bytes;
  w->ev_used = 0;
  return SPEC_OK;
}

size_t spec_workspace_size(spec_weights_t w, int32_t B, int32_t gamma) {
  if (!w || B < 1 || gamma < 0 || gamma > kMaxGamma) return 0;
  return make_layout(w, B, gamma).total;
}

spec_status spec_verify(spec_weights_t w, int32_t B, int32_t gamma, const float* hidden,
                        const int32_t* draft_tokens, const float* q, float temperature,
                        float top_p, uint64_t seed, int32_t* n_accepted, int32_t* emitted,
                        void* workspace, size_t workspace_bytes, void* stream) {
  return verify_impl(w, B, gamma, hidden, draft_tokens, q, temperature, top_p, seed, n_accepted,
                     emitted, workspace, workspace_bytes, stream, nullptr, nullptr, nullptr);
}

spec_status spec_verify_noalloc(spec_weights_t w, int32_t B, int32_t gamma, const float* hidden,
                                const int32_t* draft_tokens, const float* q, float temperature,
                                float top_p, uint64_t seed, int32_t* n_accepted, int32_t* emitted,
                                void* stream) {
  return verify_impl(w, B, gamma, hidden, draft_tokens, q, temperature, top_p, seed, n_accepted,
                     emitted, nullptr, 0, stream, nullptr, nullptr, nullptr, true);
}

spec_status spec_verify_tree_greedy(spec_weights_t w, int32_t B, int32_t n_nodes,
                                    const float* hidden, const int32_t* parent,
                                    const int32_t* tokens, int32_t* n_accepted, int32_t* emitted,
                                    int32_t* path, void* workspace, size_t workspace_bytes,
                                    void* stream, float* logits_out) {
  TreeArgs t;
  t.parent = parent; t.tokens = tokens; t.path = path;
  return verify_impl(w, B, n_nodes, hidden, nullptr, nullptr, 0.0f, 1.0f, 0, n_accepted, emitted,
                     workspace, workspace_bytes, stream, logits_out, nullptr, nullptr, false, &t);
}

spec_status spec_verify_debug(spec_weights_t w, int32_t B, int32_t gamma, const float* hidden,
                              const int32_t* draft_tokens, const float* q, float temperature,
                              float top_p, uint64_t seed, int32_t* n_accepted, int32_t* emitted,
                              void* workspace, size_t workspace_bytes, void* stream,
                              float* logits_out, float* p_out, float* q_out) {
  return verify_impl(w, B, gamma, hidden, draft_tokens, q, temperature, top_p, seed, n_accepted,
                     emitted, workspace, workspace_bytes, stream, logits_out, p_out, q_out);
}

spec_status spec_diag_access_check(int32_t d, int32_t ffn, int32_t n_blocks, int32_t vocab,
                                   int32_t wdtype, int32_t mfma_min_rows, uint32_t flags,
                                   int32_t B, int32_t gamma, int32_t shrink_bytes, char* msg,
                                   size_t msg_len, int64_t* checks) {
  if (msg && msg_len) msg[0] = 0;
  if (shrink_bytes < 0) return SPEC_EINVAL;
  if (d < 1 || ffn < 1 || n_blocks < 0 || vocab < 1 || B < 1 || gamma < 0 || gamma > kMaxGamma)
    return SPEC_EINVAL;
  if (wdtype != SPEC_F32 && wdtype != SPEC_BF16) return SPEC_EDTYPE;
  // shapes only: no device memory is touched
  spec_weights w;
  w.d = d; w.ffn = ffn; w.n_blocks = n_blocks; w.V = vocab; w.wdtype = wdtype; w.flags = flags;
  w.mfma_min_rows = mfma_min_rows > 0 ? mfma_min_rows : kDefaultMfmaMinRows;
  auto shape = [&](Mat& m, int K, int N) {
    m.K = K; m.N = N; m.Kp = roundup(K, kKStep); m.Np = roundup(N, kGroupCols);
    if (wdtype == SPEC_BF16) m.nt = mfma_block_tiles(m.Np);
    if (wdtype == SPEC_BF16 && ((flags & SPEC_FLAG_KEEP_ROWMAJOR) || w.mfma_min_rows > 1))
      m.rowmajor = reinterpret_cast<void*>(uintptr_t{256});   // marks a row-major copy; never read
  };
  w.up.resize(n_blocks);
  w.down.resize(n_blocks);
  for (int l = 0; l < n_blocks; ++l) { shape(w.up[l], d, ffn); shape(w.down[l], ffn, d); }
  shape(w.lm, d, vocab);
  AccessCheck C;
  C.msg = msg; C.msg_len = msg_len;
  const spec_status s = access_check_pass(&w, B, gamma, shrink_bytes, C);
  for (auto& m : w.up) m.rowmajor = nullptr;
  for (auto& m : w.down) m.rowmajor = nullptr;
  w.lm.rowmajor = nullptr;
  if (checks) *checks = C.checks;
  return s;
}

spec_status spec_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes == 0 || (bytes & 15) || (reinterpret_cast<uintptr_t>(src) & 15))
    return SPEC_EINVAL;
  (void)hipGetLastError();
  return launch_stream_read(src, bytes, 0x9E3779B9u, sink, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? SPEC_OK
             : SPEC_EHIP;
}

size_t spec_workspace_size_from_logits(int32_t B, int32_t gamma, int32_t vocab) {
  if (B < 1 || gamma < 0 || gamma > kMaxGamma || vocab < 1) return 0;
  Layout L;
  L.M = B * (gamma + 1);
  size_t off = 0;
  layout_sampling(L, B, gamma, vocab, (vocab + 4 * kSub - 1) / (4 * kSub), off);
  return off;
}

spec_status spec_verify_from_logits(int32_t B, int32_t gamma, int32_t vocab, const float* logits,
                                    const int32_t* draft_tokens, const float* q,
                                    float temperature, float top_p, uint64_t seed,
                                    int32_t* n_accepted, int32_t* emitted, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  if (B < 1 || gamma < 0 || gamma > kMaxGamma || vocab < 1 || !logits || !n_accepted || !emitted)
    return SPEC_EINVAL;
  if (gamma > 0 && !draft_tokens) return SPEC_EINVAL;
  if (bad_scalars(temperature, top_p)) return SPEC_EINVAL;
  if (temperature > 0.f && gamma > 0 && !q) return SPEC_EINVAL;
  Layout L;
  L.M = B * (gamma + 1);
  size_t off = 0;
  layout_sampling(L, B, gamma, vocab, (vocab + 4 * kSub - 1) / (4 * kSub), off);
  if (!workspace || workspace_bytes < off || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return SPEC_EWORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int tmode = tmode_of(temperature);
  SampleArgs sa;
  sa.B = B; sa.gamma = gamma; sa.V = vocab; sa.G = L.G; sa.Gu = L.Gu; sa.M = L.M;
  sa.logits = logits; sa.ldl = vocab; sa.q = q; sa.draft = draft_tokens;
  sa.T = temperature; sa.invT = tmode ? 1.0f / temperature : 1.0f; sa.top_p = top_p;
  sa.tmode = tmode; sa.seed = seed;
  sa.n_acc = n_accepted; sa.emitted = emitted;
  sa.pst = at<float>(workspace, L.pst); sa.pidx = at<int>(workspace, L.pidx);
  sa.qst = at<float>(workspace, L.qst); sa.rowinfo = at<float>(workspace, L.rowinfo);
  sa.dec = at<int>(workspace, L.dec); sa.csum = at<double>(workspace, L.csum); sa.nch = L.nch;
  hipError_t err = launch_tile_stats(sa, st);
  if (err == hipSuccess) err = launch_sampling(sa, st);
  return err == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

}  // extern "C"
