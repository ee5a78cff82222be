/*
 * specverify.h -- C ABI of the speculative-decoding target-verification step
 * for AMD Instinct MI355X (gfx950).
 *
 * One call scores gamma drafted positions plus the bonus position of B
 * sequences in a single pass over the target's weights, then applies the
 * acceptance rule over the vocabulary:
 *   - accept draft x_i when r_i * q'_i(x_i) < p'_i(x_i), r_i uniform in [0,1)
 *     ("Speculative decoding" explainer, lattice-ai-eng.pages.dev: acceptance
 *     rule; pigeon guide "Speculative decoding", How it works, step 3);
 *   - at the first rejection j, sample a replacement from
 *     norm(max(0, p'_j - q'_j)) and drop the later drafts (pigeon guide, step
 *     4), or from p'_j when that residual is exactly zero ("Build a
 *     Speculative Decoding Engine to Cut LLM Latency by 3x", The Accept/Reject
 *     Mechanism, numerical fallback);
 *   - if nothing is rejected, sample one bonus token from p'_gamma (pigeon
 *     guide, step 5);
 *   - at temperature 0, accept while the draft equals the target's argmax and
 *     emit the argmax (lattice-ai-eng explainer, greedy remark).
 * p' and q' are the target and draft distributions after the same
 * temperature and top-p transform (pigeon guide, When it breaks; scalablesystem
 * article, Quality, Evaluation, and Guardrails, item 1).  q' is q^(1/T)
 * renormalised; the nucleus is the shortest prefix of the tokens sorted by
 * probability (descending, ties by lower id) whose mass reaches top_p.
 *
 * Sampling uses the inverse CDF in token-id order (smallest v whose inclusive
 * prefix sum exceeds u * total).  Uniforms come from Philox4x64-10 (Salmon et
 * al., SC'11) with key (seed, 0) and counter (i, b, 0, 0): r_{b,i} is the top
 * 24 bits of word 0 times 2^-24 and u_{b,i} the top 24 bits of word 1, so a
 * run is reproducible from its seed (scalablesystem article, guardrail 3).
 *
 * The synthetic target is a stack of MLP blocks
 *     n = h / sqrt(mean(h^2) + eps) * g;  h += SiLU(n @ W_up) @ W_down
 * followed by logits = h @ W_lm (no final norm).  Weights are row-major
 * [in][out].
 *
 * Conventions for every entry point:
 *   - Pointers documented "device" are HIP device pointers; "host" pointers
 *     are ordinary process memory.  The caller owns every buffer it passes.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means
 *     the default stream).  The caller synchronises the stream before it
 *     reads outputs.
 *   - Shapes, scalars, pointers and workspace size are checked before any
 *     launch; on error nothing is launched and a negative spec_status is
 *     returned.  A row whose draft token id lies outside [0, vocab) gets
 *     n_accepted = -1 and an all -1 emitted row; other rows are unaffected.
 *   - Non-finite inputs are a precondition violation: no fault, unspecified
 *     outputs.
 *   - Calls that share a workspace must not overlap in time.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPEC_OK = 0,
  SPEC_EINVAL = -1,      /* bad shape, scalar or null pointer              */
  SPEC_EDTYPE = -2,      /* unsupported weight dtype                       */
  SPEC_EWORKSPACE = -3,  /* workspace missing or smaller than required     */
  SPEC_EHIP = -4,        /* a HIP runtime call failed                      */
  SPEC_ENOMEM = -5,      /* device allocation failed (create only)         */
  SPEC_ESCRATCH = -6     /* pass larger than SPEC_NOALLOC_SCRATCH_BYTES
                            (spec_verify_noalloc only)                     */
} spec_status;

typedef enum { SPEC_F32 = 0, SPEC_BF16 = 1 } spec_dtype;

/* Flags for spec_weights_desc.flags. */
#define SPEC_FLAG_KEEP_ROWMAJOR 1u  /* bf16: also keep a row-major copy so the
                                       vector-FMA GEMM can serve any row count */
#define SPEC_FLAG_EXACT_SPLIT 2u    /* bf16: keep the exact three-term split
                                       of each fp32 activation in every pass.
                                       Without it, passes of 9 to 224 rows
                                       (the wide GEMM's) and of 6 to 8 rows
                                       carry each activation as two bf16
                                       terms rounded to nearest (|x - hi -
                                       lo| <= 2^-16 |x|): a third fewer
                                       matrix operations, LDS reads and
                                       activation bytes per k-step, or eight
                                       rows in one stacked fragment instead
                                       of five, at a logit error about 1.5 to
                                       10 times the exact split's (measured
                                       under 1e-5 of max |logit|).  Passes of
                                       up to 5 rows keep three terms. */

/* Description of the target's weights, read once by spec_weights_create.
 * The pointer arrays are host arrays of n_blocks device pointers.  The
 * library copies (and repacks) every weight into memory it owns, so the
 * caller may free its buffers once spec_weights_create has returned and the
 * stream has been synchronised. */
typedef struct {
  int32_t d;               /* hidden size                                  */
  int32_t ffn;             /* MLP inner size                               */
  int32_t n_blocks;        /* number of MLP blocks (>= 0)                  */
  int32_t vocab;           /* V                                            */
  int32_t wdtype;          /* spec_dtype of every weight and gain          */
  float rms_eps;           /* RMSNorm epsilon (1e-6 in the workloads)      */
  const void* const* w_up;      /* host array: n_blocks device [d][ffn]    */
  const void* const* w_down;    /* host array: n_blocks device [ffn][d]    */
  const void* const* norm_gain; /* NULL (all ones) or host array of
                                   n_blocks device [d]                     */
  const void* lm_head;          /* device [d][vocab]                       */
  uint32_t flags;               /* SPEC_FLAG_*                             */
  int32_t mfma_min_rows;        /* bf16: use the MFMA GEMM when
                                   B*(gamma+1) >= this; <= 0 means the
                                   library default                         */
} spec_weights_desc;

typedef struct spec_weights* spec_weights_t;

/* Validate the description, allocate device memory and copy the weights
 * into the library's layouts (fp32 row-major for SPEC_F32; MFMA tiles for
 * SPEC_BF16, plus row-major when SPEC_FLAG_KEEP_ROWMAJOR).  Runs on `stream`
 * and synchronises it before returning.  *out is set only on SPEC_OK. */
spec_status spec_weights_create(const spec_weights_desc* desc, void* stream,
                                spec_weights_t* out);

/* Free what spec_weights_create allocated.  NULL is accepted. */
spec_status spec_weights_destroy(spec_weights_t w);

/* Bytes of device workspace spec_verify / spec_verify_debug need for this
 * batch shape, or 0 when the arguments are invalid (B < 1, gamma < 0). */
size_t spec_workspace_size(spec_weights_t w, int32_t B, int32_t gamma);

/* The verification step.
 *   hidden       device fp32 [B][gamma+1][d]; row i < gamma scores draft i,
 *                row gamma scores the bonus slot
 *   draft_tokens device int32 [B][gamma]
 *   q            device fp32 [B][gamma][vocab], the draft's temperature-1
 *                probabilities (need not be normalised; not read when
 *                temperature == 0, may then be NULL)
 *   temperature  >= 0 and finite; 0 selects the greedy rule
 *   top_p        in (0, 1]; 1 disables the nucleus; ignored when
 *                temperature == 0
 *   seed         Philox key word 0
 *   n_accepted   device int32 [B] out: 0..gamma, or -1 for a bad row
 *   emitted      device int32 [B][gamma+1] out: the n accepted drafts, then
 *                the correction or bonus token, then -1 padding
 *   workspace    device, at least spec_workspace_size(w, B, gamma) bytes,
 *                256-byte aligned; contents on entry are ignored */
spec_status spec_verify(spec_weights_t w, int32_t B, int32_t gamma,
                        const float* hidden, const int32_t* draft_tokens,
                        const float* q, float temperature, float top_p,
                        uint64_t seed, int32_t* n_accepted, int32_t* emitted,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Scratch bytes the allocation-free entry point holds per GPU. */
#define SPEC_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/* spec_verify for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It takes no workspace: the pass runs in a static per-GPU scratch array of
 * SPEC_NOALLOC_SCRATCH_BYTES (128 MiB; reserved in each GPU's memory the
 * library runs on until the process ends), whose address the library looks
 * up once per device in spec_weights_create.  The call allocates nothing
 * (no hipMalloc, hipFree, event creation or allocating library routine);
 * timing (spec_profile_enable) does not apply to it.  The caller still
 * passes inputs and outputs, as for spec_verify.  Every call on a GPU
 * shares that GPU's scratch and leaves its contents behind (the kernels
 * read no workspace content they have not written in the same call), so
 * calls that overlap in time on one GPU, on any streams, race: serialise
 * them.  Returns SPEC_ESCRATCH, before any launch, when
 * spec_workspace_size(w, B, gamma) exceeds the scratch; other arguments and
 * errors as for spec_verify. */
spec_status spec_verify_noalloc(spec_weights_t w, int32_t B, int32_t gamma,
                                const float* hidden, const int32_t* draft_tokens,
                                const float* q, float temperature, float top_p,
                                uint64_t seed, int32_t* n_accepted, int32_t* emitted,
                                void* stream);

/* spec_verify plus optional dumps for parity checks (not a timed path).
 *   logits_out  device fp32 [B][gamma+1][vocab] or NULL: target logits
 *   p_out       device fp32 [B][gamma+1][vocab] or NULL: p' (T > 0 only)
 *   q_out       device fp32 [B][gamma][vocab] or NULL: q' (T > 0 only) */
spec_status spec_verify_debug(spec_weights_t w, int32_t B, int32_t gamma,
                              const float* hidden, const int32_t* draft_tokens,
                              const float* q, float temperature, float top_p,
                              uint64_t seed, int32_t* n_accepted,
                              int32_t* emitted, void* workspace,
                              size_t workspace_bytes, void* stream,
                              float* logits_out, float* p_out, float* q_out);

/* Greedy verification of a draft tree ("Speculative Decoding: Speeding
 * Sequential Generation", aicomputerinstitute.com, Tree-Based Drafting,
 * Constructing the Tree Attention Mask in Code, Expected Tokens per
 * Verification Round: Chain vs. Tree).  One pass scores the root row and
 * one row per node; node j passes when its token equals the argmax of its
 * parent's row (temperature 0).  From the root, the walk descends to the
 * lowest-index passing child until a row has none, and emits that row's
 * argmax (correction, or bonus at a leaf).  The synthetic target has no
 * attention, so node rows are scored independently: a caller whose model
 * attends builds the node rows with the tree mask (node i sees itself and
 * its ancestors) and position id = depth before this call.
 *   hidden      device fp32 [B][n_nodes+1][d]: row 0 the root (the last
 *               committed position), row 1 + j node j
 *   parent      device int32 [B][n_nodes]: -1 for a child of the root, else
 *               a node index below j (parents precede children)
 *   tokens      device int32 [B][n_nodes]: the draft token of each node
 *   n_accepted  device int32 [B] out: depth of the accepted path, or -1
 *               when a parent or token of the sequence is out of range
 *   emitted     device int32 [B][n_nodes+1] out: the accepted path's tokens,
 *               then the argmax of its last row, then -1 padding
 *   path        device int32 [B][n_nodes] out or NULL: node indices of the
 *               accepted path, -1 padding (what a KV cache commits)
 *   workspace   spec_workspace_size(w, B, n_nodes) bytes (a pass of
 *               n_nodes + 1 rows per sequence), 256-byte aligned
 *   logits_out  device fp32 [B][n_nodes+1][vocab] or NULL (parity checks)
 * Ties: the lowest token id for an argmax, the lowest node index among
 * children with equal tokens. */
spec_status spec_verify_tree_greedy(spec_weights_t w, int32_t B, int32_t n_nodes,
                                    const float* hidden, const int32_t* parent,
                                    const int32_t* tokens, int32_t* n_accepted,
                                    int32_t* emitted, int32_t* path, void* workspace,
                                    size_t workspace_bytes, void* stream, float* logits_out);

/* Workspace bytes for spec_verify_from_logits, or 0 on invalid arguments. */
size_t spec_workspace_size_from_logits(int32_t B, int32_t gamma, int32_t vocab);

/* The acceptance rule alone, given target logits instead of hidden states
 * and weights: logits is device fp32 [B][gamma+1][vocab].  Every other
 * argument means what it means for spec_verify. */
spec_status spec_verify_from_logits(int32_t B, int32_t gamma, int32_t vocab,
                                    const float* logits,
                                    const int32_t* draft_tokens,
                                    const float* q, float temperature,
                                    float top_p, uint64_t seed,
                                    int32_t* n_accepted, int32_t* emitted,
                                    void* workspace, size_t workspace_bytes,
                                    void* stream);

/* Kernel timing for benchmarks.  While enabled, every GEMM launch that
 * spec_verify / spec_verify_debug make with these weights carries a pair of
 * HIP events that take the kernel's own start and end timestamps
 * (hipExtLaunchKernel; the library creates the events, and a call may grow
 * the pool).  spec_profile_read synchronises those
 * events and returns, since the previous read or enable: the summed GEMM
 * time in milliseconds, the number of GEMM launches, and the algorithmic
 * weight bytes they streamed (K * N * bytes per weight, padding excluded);
 * any out pointer may be NULL.  Reading clears the record. */
spec_status spec_profile_enable(spec_weights_t w, int32_t on);
spec_status spec_profile_read(spec_weights_t w, double* gemm_ms, int64_t* launches,
                              int64_t* weight_bytes);

/* Streaming-read probe for benchmarks: one launch that reads `bytes` from
 * the device buffer `src` with 16-byte non-temporal loads (the access the
 * weight-streaming GEMMs make) and discards them, so that the time of a
 * launch gives the read bandwidth this device reaches for that size.
 *   src    device, 16-byte aligned, `bytes` readable (a multiple of 16)
 *   sink   device uint32 the kernel may write (it does only when the folded
 *          words hit a fixed key); owned by the caller
 * Asynchronous on `stream`; SPEC_EINVAL for a null pointer, zero or
 * unaligned size. */
spec_status spec_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* ---- Host policy around the step ("Build a Speculative Decoding Engine
 * to Cut LLM Latency by 3x", scalablesystem.dev, Dynamic Gamma Controller
 * and Batch-Level Speculation). */

/* Speculation-depth controller for n_seq sequences (host memory only, no
 * GPU work).  Each sequence keeps the last 20 (accepted, rejected) counts,
 * rejected = gamma used - accepted; its rolling acceptance rate is
 * sum(accepted) / sum(accepted + rejected) (0.80 before any step).  From 5
 * recorded steps on, each update sets its gamma to the value in
 * [gamma_min, gamma_max] maximising
 *     E(g) / (g * draft_ms_per_token + target_ms[g]),
 *     E(g) = (1 - alpha^(g+1)) / (1 - alpha)   (g + 1 at alpha = 1),
 * the smallest such g on ties.
 *   target_ms  host [gamma_max + 1]: verification time of a pass with g
 *              drafts (entries gamma_min .. gamma_max read, each > 0); a
 *              constant array gives the article's fixed target time
 * SPEC_EINVAL for bad bounds or times; *out set on SPEC_OK. */
typedef struct spec_gamma_ctl* spec_gamma_ctl_t;
spec_status spec_gamma_ctl_create(int32_t n_seq, int32_t gamma_min, int32_t gamma_max,
                                  int32_t gamma_init, double draft_ms_per_token,
                                  const double* target_ms, spec_gamma_ctl_t* out);
spec_status spec_gamma_ctl_destroy(spec_gamma_ctl_t c);

/* Record one step of every sequence and return the gamma of its next step.
 *   n_accepted  host [n_seq]: the step's n_accepted (-1: refused row, which
 *               records nothing)
 *   gamma_used  host [n_seq]: the gamma each sequence was verified with
 *   gamma_next  host [n_seq] out
 * SPEC_EINVAL (nothing recorded) when some n_accepted exceeds its gamma. */
spec_status spec_gamma_ctl_update(spec_gamma_ctl_t c, const int32_t* n_accepted,
                                  const int32_t* gamma_used, int32_t* gamma_next);

/* Rolling acceptance rate of sequence seq (-1 for a bad index). */
double spec_gamma_ctl_alpha(spec_gamma_ctl_t c, int32_t seq);

/* The gamma the controller picks for acceptance rate alpha in [0, 1]
 * (-1 for a bad alpha). */
int32_t spec_gamma_ctl_optimal(spec_gamma_ctl_t c, double alpha);

/* Ragged repacking after a verification step of B sequences, on the device
 * (one work group, asynchronous on `stream`, no host round trip).  Row b
 * emitted count_b = n_accepted[b] + 1 tokens when 0 <= n_accepted[b] <=
 * gamma, else none (a refused row).  All pointers are device memory:
 *   n_accepted   int32 [B], emitted int32 [B][gamma+1] (spec_verify's outputs)
 *   committed    int32 [B] in/out: committed length, advanced by count_b
 *   tokens       int32 [B*(gamma+1)] out: the emitted tokens, rows end to end
 *   offsets      int32 [B+1] out: row b's tokens are tokens[offsets[b] ..
 *                offsets[b+1])
 *   order        int32 [B] out: sequence ids sorted by count, stably (ids
 *                ascending within a count): micro-batches by accepted count
 *   bin_offsets  int32 [gamma+3] out: sequences with count c are
 *                order[bin_offsets[c] .. bin_offsets[c+1]), c = 0 .. gamma+1
 *   stats        int32 [2] out: padded width max(count) of one padded batch,
 *                and its waste B * width - sum(count)
 * SPEC_EINVAL for B < 1, gamma < 0, gamma > 254 or a null pointer. */
spec_status spec_repack(int32_t B, int32_t gamma, const int32_t* n_accepted,
                        const int32_t* emitted, int32_t* committed, int32_t* tokens,
                        int32_t* offsets, int32_t* order, int32_t* bin_offsets, int32_t* stats,
                        void* stream);

/* ---- Attention of the verification pass's new rows over a KV-cached
 * prefix, and the commit of the accepted rows ("Build a Speculative
 * Decoding Engine to Cut LLM Latency by 3x", scalablesystem.dev, KV Cache
 * Management for Dual Models and Rollback Protocol; "Speculative Decoding:
 * Speeding Sequential Generation", aicomputerinstitute.com, Constructing
 * the Tree Attention Mask in Code).
 *
 * Cache layout (device, bf16 bits): k_cache [B][Hkv][max_seq][hd] (a key's
 * head dimension contiguous) and v_cache [B][Hkv][hd][max_seq] (values
 * head-dimension major, so eight consecutive positions of one dimension
 * are one 16-byte MFMA operand); max_seq a multiple of 8.
 * Sequence b has cache_len[b] committed positions; the keys and values of
 * its n_new new rows (the root, then the drafts in chain or tree order,
 * already projected and position-encoded by the caller, position id =
 * depth) sit at slots cache_len[b] .. cache_len[b] + n_new - 1.  A
 * cache_len outside [0, max_seq - n_new] is clamped into it. */

/* Workspace bytes of spec_decode_attention, 0 for invalid shapes. */
size_t spec_attention_workspace_size(int32_t B, int32_t n_new, int32_t H, int32_t Hkv,
                                     int32_t head_dim, int32_t max_seq);

/* out[b][i][h][:] = sum_t softmax_t(scale * q[b][i][h] . k[b][kv][t]) v[b][kv][t]
 * over the slots new row i sees: every committed slot, itself, and its
 * ancestors among the new rows; kv = h / (H / Hkv) (grouped-query heads).
 *   q          device fp32 [B][n_new][H][hd]
 *   cache_len  device int32 [B]
 *   parent     device int32 [B][n_new] or NULL: the parent of each new row
 *              among the new rows (-1: none; parents precede children, a
 *              value outside [-1, i) counts as -1); NULL is a chain
 *              (parent i - 1), i.e. the causal mask
 *   out        device fp32 [B][n_new][H][hd]
 *   workspace  spec_attention_workspace_size bytes, 256-byte aligned
 * Shapes: 1 <= n_new <= 64, H a multiple of Hkv, hd 64 or 128, max_seq a
 * multiple of 8, caches 16-byte aligned; SPEC_EINVAL / SPEC_EWORKSPACE
 * otherwise.  Both products run on bf16 MFMA: the queries (times
 * scale * log2(e), the softmax running in base 2) split into three bf16
 * terms (exact), the probabilities into two (2^-16 relative).  Results are
 * run-to-run identical (no atomics; partials merged in a fixed order). */
spec_status spec_decode_attention(int32_t B, int32_t n_new, int32_t H, int32_t Hkv,
                                  int32_t head_dim, int32_t max_seq, const float* q,
                                  const uint16_t* k_cache, const uint16_t* v_cache,
                                  const int32_t* cache_len, const int32_t* parent, float scale,
                                  float* out, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* Commit one step: keep the root and the n_accepted[b] accepted rows, drop
 * the rest by not moving past them (the memory is reused next step).  With
 * path (device int32 [B][n_new - 1], the accepted nodes of a tree walk,
 * node j being new row j + 1), the accepted rows' keys and values are first
 * gathered to slots cache_len[b] + 1 .. cache_len[b] + n_accepted[b] for
 * every KV head (caches in the layout above); path NULL is a chain, whose
 * accepted rows already sit
 * there (k_cache and v_cache may then be NULL).  Then cache_len[b] +=
 * n_accepted[b] + 1 on the device; a row with n_accepted < 0 is left alone. */
spec_status spec_kv_commit(int32_t B, int32_t n_new, int32_t Hkv, int32_t head_dim,
                           int32_t max_seq, uint16_t* k_cache, uint16_t* v_cache,
                           int32_t* cache_len, const int32_t* n_accepted, const int32_t* path,
                           void* stream);

/* Static text for a status code. */
const char* spec_status_string(spec_status s);

/* Row count B*(gamma+1) from which bf16 weights use the MFMA GEMM when the
 * description leaves mfma_min_rows at 0. */
int32_t spec_default_mfma_min_rows(void);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
