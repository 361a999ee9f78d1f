/*
 * sparse_attn.h -- C ABI of the block-sparse causal prefill attention library (gfx950).
 *
 * The method, in the order the calls run it:
 *
 *   sparse_attn_score    Block summaries of the keys: mean-pooled keys or per-coordinate
 *                        K-min/K-max bounds, plus the mean value-row L2 norm when the
 *                        output-aware score is on.  ("Uncertainty-Gated Selection for
 *                        Block-Sparse Attention" page, Metodologia step 1; Stem page,
 *                        Metodologia B and the three-stage implementation note.)
 *   sparse_attn_select   Per query tile and head: tile score = max over the tile's rows,
 *                        top-k under a constant or position-decaying budget, the normalised
 *                        cut margin sigma = (s_(k-1) - s_(k)) / (s_(0) - s_(k)), its mean
 *                        over heads, a per-call quantile gate, top-floor(rho*k) expansion of
 *                        tripped tiles, and sentinel-padded block lists.  (Gated-selection
 *                        page, Metodologia steps 2-5; Stem page, Metodologia A.)
 *   sparse_attn_forward  FlashAttention-style online-softmax attention over the listed KV
 *                        blocks only, causal.  (Stem page, implementation note; ART page,
 *                        section 2.4 on order invariance of the online softmax.)
 *
 * Conventions shared by every call:
 *   - Q is [B, N, Hq, d], K and V are [B, N, Hkv, d], O is [B, N, Hq, d]: contiguous, row
 *     major (BSHD).  Query head h reads kv head h / (Hq / Hkv).
 *   - Every pointer argument is device memory allocated and owned by the caller; the
 *     library never allocates, frees or keeps a pointer after a call returns.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue work and
 *     return; results are ready when the stream is.  A fault inside a kernel surfaces at the
 *     caller's next synchronisation of that stream.
 *   - Return value: SA_OK, or a negative status.  Arguments are validated on the host
 *     before any HIP call, so an invalid call enqueues nothing.  sparse_attn_last_error()
 *     gives the calling thread's last message.
 *   - Supported in this version: head_dim in {64, 128}; block == tile in {64, 128}, or
 *     tile 128 over block 64;
 *     seqlen % block == 0; Hq % Hkv == 0; bf16 or fp32 inputs; at most 16384 blocks per
 *     sequence, within the selection's LDS limit (sparse_attn_select).
 */
#ifndef SPARSE_ATTN_H_
#define SPARSE_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SA_OK = 0,
  SA_ERR_INVALID = -1,     /* bad argument: null pointer, out-of-range value, small buffer */
  SA_ERR_UNSUPPORTED = -2, /* valid but not supported by this library version (shape, dtype) */
  SA_ERR_HIP = -3          /* a HIP call failed (launch, device query) */
};

enum { SA_F32 = 0, SA_BF16 = 1 };                            /* element types */
enum { SA_KMEAN = 0, SA_KMINMAX = 1 };                       /* block score backbones */
enum { SA_K_CONST = 0, SA_K_LINEAR_DECAY = 1 };              /* budget schedules */
enum { SA_GATE_QUANTILE = 0, SA_GATE_FIXED = 1, SA_GATE_OFF = 2 }; /* gate threshold source */
enum { SA_OAM_OFF = 0, SA_OAM_PRODUCT = 1, SA_OAM_ADDITIVE = 2 };   /* output-aware scoring */
enum { SA_SELECT_PER_Q_HEAD = 0, SA_SELECT_PER_KV_HEAD = 1 };       /* one list per ... */

/* Shapes and scoring mode. */
typedef struct sa_problem {
  int32_t batch;        /* B >= 1 */
  int32_t seqlen;       /* N, a multiple of block */
  int32_t n_q_heads;    /* Hq, a multiple of n_kv_heads */
  int32_t n_kv_heads;   /* Hkv >= 1 */
  int32_t head_dim;     /* d: 64 or 128 */
  int32_t block;        /* key block size: 64 or 128 */
  int32_t tile;         /* query tile rows T: equal to block, or 128 over blocks of 64 (then
                           tile t's diagonal blocks 2t and 2t+1 are both forced, its free
                           blocks are 0 .. 2t-1, and n below counts tiles, N / T) */
  int32_t dtype;        /* SA_BF16 or SA_F32, for Q, K and V */
  int32_t score_mode;   /* SA_KMEAN: mean-pooled keys; SA_KMINMAX: per-coordinate bound */
  int32_t output_aware; /* SA_OAM_OFF; SA_OAM_PRODUCT: tile score times the block's mean
                           value-row L2 norm vnorm; SA_OAM_ADDITIVE (Stem page, Metodologia B):
                           fmaf(tile score, (float)(1/sqrt(d)), bonus) with
                           bonus = (float)(oam_beta * max(0, ln(vnorm^2))) in fp64 */
  float oam_beta;       /* beta of SA_OAM_ADDITIVE: finite, >= 0; ignored otherwise */
  int32_t select_unit;  /* SA_SELECT_PER_Q_HEAD: one list per query head (the gated-selection
                           page's per-head selection, Metodologia steps 2-3).
                           SA_SELECT_PER_KV_HEAD: one list per kv head, shared by its
                           Hq / Hkv query heads (a GQA variant the pages do not describe): the
                           tile score is the maximum over the tile's rows of all those heads;
                           sigma is per kv head and sigma_bar their mean.  U below is the
                           number of selection units per sequence: Hq, or Hkv. */
} sa_problem;

/* Budget, forced blocks and gate.  n = seqlen / tile query tiles per sequence (equal to the
 * number of blocks when tile = block). */
typedef struct sa_budget {
  int32_t k_max;     /* free blocks kept per tile (constant budget), or the decay's start */
  int32_t k_min;     /* floor of the decaying budget; 1 <= k_min <= k_max */
  int32_t kind;      /* SA_K_CONST: k_t = k_max; SA_K_LINEAR_DECAY:
                        k_t = max(k_min, floor(k_max * (n - t) / n)) */
  int32_t n_sink;    /* blocks 0 .. n_sink-1 are always kept (on top of k); >= 0 */
  int32_t gate_mode; /* SA_GATE_QUANTILE: tau_b = ceil(q*M_b)-th smallest sigma_bar over
                        batch element b's M_b eligible tiles; SA_GATE_FIXED: tau = tau_fixed;
                        SA_GATE_OFF: no tile trips */
  float tau_fixed;   /* threshold for SA_GATE_FIXED */
  double rho;        /* expansion factor >= 1: a tripped tile keeps floor(rho * k_t) */
  double q;          /* quantile in [0, 1] for SA_GATE_QUANTILE */
} sa_budget;

/*
 * Bytes of the block-summary buffer `sparse_attn_score` fills, for this problem.
 * It starts with (all fp32, n = seqlen / block):
 *   SA_KMEAN:   kmean [B, n, Hkv, d]
 *   SA_KMINMAX: kmin  [B, n, Hkv, d] followed by kmax [B, n, Hkv, d]
 *   then, if output_aware != SA_OAM_OFF: vnorm [B, n, Hkv]
 * and continues with auxiliary data for sparse_attn_select whose layout is private
 * (per-block norms, and bf16 and fp32 copies of the planes above in a blocked order: about
 * one and a half times as large again).
 * Returns 0 for an invalid problem (see sparse_attn_last_error).
 */
size_t sparse_attn_summary_bytes(const sa_problem* p);

/* Bytes of device workspace `sparse_attn_select` needs.  0 for invalid arguments. */
size_t sparse_attn_select_workspace_bytes(const sa_problem* p, const sa_budget* b);

/*
 * W, the entries per padded list: min(seqlen / block, tile / block + n_sink +
 * floor(rho * k_max)) (tile / block diagonal blocks).
 * Returns a negative status for invalid arguments.
 */
int32_t sparse_attn_index_width(const sa_problem* p, const sa_budget* b);

/*
 * Block summaries (gated-selection page, Metodologia step 1; Stem page, output-aware metric).
 *   K          [B, N, Hkv, d] in p->dtype.
 *   V          [B, N, Hkv, d]; read only when p->output_aware, may be NULL otherwise.
 *   summaries  sparse_attn_summary_bytes(p) bytes, written.
 * Output-aware scoring holds block * n_kv_heads fp32 norms in LDS: at most 159744 bytes,
 * else SA_ERR_UNSUPPORTED before any HIP call.
 * Per block j and kv head g: kmean = (sum of the block's key rows in row order, fp32) / block;
 * kmin/kmax = per-coordinate min/max (exact); vnorm = (sum over rows in order of the fp32
 * L2 norm of the value row) / block.
 */
int sparse_attn_score(const sa_problem* p, const void* K, const void* V, void* summaries,
                      void* stream);

/*
 * Selection (gated-selection page, Metodologia steps 2-5; Stem page, Metodologia A).
 *   Q          [B, N, Hq, d] in p->dtype.
 *   summaries  from sparse_attn_score on the same problem.
 *   ws         sparse_attn_select_workspace_bytes(p, b) bytes of scratch, contents ignored.
 *   kv_idx     int32 [B, U, n, W], W = sparse_attn_index_width(p, b), U = Hq or Hkv (see
 *              select_unit): tile t's kept blocks in ascending order (so its diagonal block or
 *              blocks come last), then -1 sentinels.
 *   kv_cnt     int32 [B, U, n]: number of non-sentinel entries.
 *   sigma      optional (NULL to skip) fp32 [B, U, n]: cut margin per tile and unit; 1.0
 *              for a tile with at most k_t free candidates (not eligible).
 *   sigma_bar  optional fp32 [B, n]: mean of sigma over the U units.
 *   gate       optional uint8 [B, n]: 1 where the tile tripped and kept floor(rho * k_t).
 *   tau        optional fp32 [B]: the threshold used (-inf when nothing can trip).
 * Free blocks of tile t are the blocks before its diagonal ones (block t, or blocks 2t and
 * 2t+1 for 128-row tiles over 64-key blocks) minus the n_sink first blocks; they rank by
 * tile score, ties to the lower index; the diagonal and sink blocks are always kept.  Scores are
 * fp32 with a fixed reduction order, so the lists are reproducible bit for bit.
 * LDS limit: one workgroup holds a sort key per block, P of them (P = n rounded up to a power
 * of two), and for bf16 inputs the tile's query rows, Qb = 2 * planes * tile * (d + 8) bytes
 * (planes = 2 for SA_KMINMAX, else 1).  Keys take 8 bytes, except with bf16 inputs when
 * 16 * pow2(Rn) <= Qb, Rn = min(max(floor(rho * k_max), k_max + 1), n) (pow2 rounds up to a
 * power of two): then 4 bytes, 4 * P rounded up to a multiple of 16.  Keys plus Qb must not
 * exceed 159744 bytes, else SA_ERR_UNSUPPORTED before any HIP call (with 4-byte keys up to
 * 16384 blocks always fit, and 32768 with SA_KMEAN and 64-row tiles; with 8-byte keys 8192).
 * sparse_attn_select_workspace_bytes returns 0 for such problems.
 */
int sparse_attn_select(const sa_problem* p, const sa_budget* b, const void* Q,
                       const void* summaries, void* ws, size_t ws_bytes, int32_t* kv_idx,
                       int32_t* kv_cnt, float* sigma, float* sigma_bar, uint8_t* gate,
                       float* tau, void* stream);

/* Bytes of device workspace `sparse_attn_forward` needs: 0 for fp32 problems; for bf16 ones
 * the size of V plus 256-byte-aligned room for 260 bytes per (batch, kv head) (the prepared
 * values below).  0 also for an invalid problem (see sparse_attn_last_error). */
size_t sparse_attn_forward_workspace_bytes(const sa_problem* p);

/*
 * Sparse attention (Stem page, three-stage implementation; gated-selection page, step 5).
 *   Q, K, V        BSHD in p->dtype.
 *   kv_idx, kv_cnt [B, U, n, W] and [B, U, n] as written by sparse_attn_select for the same
 *                  select_unit (query head h reads unit h, or its kv head h / (Hq / Hkv));
 *                  any order of blocks is accepted; the
 *                  list of query tile t ends at kv_cnt or at the first negative entry;
 *                  entries must be distinct causal blocks of the tile (<= its last
 *                  diagonal block), others are skipped).
 *   W              row stride of kv_idx (its last dimension), >= 1.
 *   softmax_scale  logit scale, normally 1/sqrt(d).
 *   ws             sparse_attn_forward_workspace_bytes(p) bytes of scratch (may be NULL when
 *                  that is 0); its contents are ignored and overwritten.
 *   O              [B, N, Hq, d] in out_dtype (SA_BF16 or SA_F32), written.
 *   lse            optional fp32 [B, Hq, N]: natural-log log-sum-exp of the scaled logits.
 * Row i of tile t attends to every key of its listed blocks at a position <= i.
 * Precision: fp32 accumulation.  With bf16 inputs, Q K^T runs on bf16 matrix cores and P V on
 * fp16 ones: P is rounded to fp16 (11 significant bits), and V, per (batch, kv head), is
 * multiplied by the power of two 2^e that brings its largest magnitude into [2^14, 2^15),
 * converted to fp16, and the outputs multiplied by 2^-e.  Every finite bf16 V is accepted:
 * values within a factor 2^29 of their head's largest magnitude convert exactly, smaller ones
 * with an absolute error below 2^-25 * 2^-e.  The error of O therefore scales with the
 * magnitude of V.  fp32 inputs are computed in fp32 throughout.
 * Limit: with bf16 inputs, seqlen * n_kv_heads * head_dim * 2 (the bytes of K per batch
 * element) must be below 2^32, else SA_ERR_UNSUPPORTED.
 * With bf16 inputs this call is sparse_attn_prepare_values followed by
 * sparse_attn_forward_prepared on the same workspace.
 */
int sparse_attn_forward(const sa_problem* p, const void* Q, const void* K, const void* V,
                        const int32_t* kv_idx, const int32_t* kv_cnt, int32_t W,
                        float softmax_scale, void* ws, size_t ws_bytes, void* O,
                        int32_t out_dtype, float* lse, void* stream);

/*
 * The two halves of sparse_attn_forward for bf16 problems, for callers that reuse one V across
 * several attention calls or time the attention kernel on its own (SA_ERR_UNSUPPORTED for
 * fp32 problems, whose forward pass reads V directly).
 *
 * sparse_attn_prepare_values: V [B, N, Hkv, d] bf16 -> ws (sparse_attn_forward_workspace_bytes
 *   bytes): the largest magnitude of each (batch, kv head), its power-of-two exponent e, and V
 *   times 2^e as fp16 in the attention kernel's transposed 32-key step layout (private).
 * sparse_attn_forward_prepared: the attention of sparse_attn_forward, reading V from a
 *   workspace that sparse_attn_prepare_values filled for the same problem and the same V
 *   (stream order makes that call's results visible; another V gives another V's attention).
 *   Other arguments and results as for sparse_attn_forward.
 */
int sparse_attn_prepare_values(const sa_problem* p, const void* V, void* ws, size_t ws_bytes,
                               void* stream);
int sparse_attn_forward_prepared(const sa_problem* p, const void* Q, const void* K,
                                 const void* ws, size_t ws_bytes, const int32_t* kv_idx,
                                 const int32_t* kv_cnt, int32_t W, float softmax_scale, void* O,
                                 int32_t out_dtype, float* lse, void* stream);

/*
 * A threshold for SA_GATE_FIXED calibrated on sample inputs.  The gated-selection page
 * (Metodologia step 4) gates each layer at an empirical quantile of sigma_bar; this call turns
 * the per-sequence thresholds sparse_attn_select wrote (tau, [batch] fp32, from calibration
 * inputs run with SA_GATE_QUANTILE) into one per-layer threshold: the mean of the finite
 * entries (an fp32 sum in index order divided by their count), or -inf when none is finite
 * (nothing could trip).  tau_out: one fp32, written.  Device pointers; one tiny kernel.
 */
int sparse_attn_calibrate_tau(const float* tau, int32_t batch, float* tau_out, void* stream);

/*
 * Sparse attention over a vertical-slash index (VSPrefill page, Metodologia B.3: the fused
 * kernel merges the vertical and the slash indices on the fly, with Merge Path, instead of
 * reading per-tile lists).  Block granularity: query tile t reads
 *   the vertical key blocks v <= t,  the blocks t - delta for the slash offsets delta <= t,
 *   and its diagonal block t,
 * each block once, then attends exactly as sparse_attn_forward does over that list.
 *   vertical   int32 [B, Hq, n_vertical]: key-block indices per query head, ascending and
 *              distinct; the list ends at n_vertical or at its first negative entry.
 *   slash      int32 [B, Hq, n_slash]: block offsets >= 0 per query head, ascending and
 *              distinct; same end rule.  (Offset 0, the diagonal, is implied.)
 *   n_vertical, n_slash >= 0 with n_vertical + n_slash <= 511, else SA_ERR_UNSUPPORTED.
 *   Other arguments as for sparse_attn_forward; ws is required.
 * bf16 inputs only (SA_ERR_UNSUPPORTED otherwise).  Indices that break the ascending-and-
 * distinct contract give wrong lists, never an access outside the tile's causal blocks.
 * The indices come from the caller (the pages' trained indexer, or any other source).
 */
int sparse_attn_forward_vs(const sa_problem* p, const void* Q, const void* K, const void* V,
                           const int32_t* vertical, int32_t n_vertical, const int32_t* slash,
                           int32_t n_slash, float softmax_scale, void* ws, size_t ws_bytes,
                           void* O, int32_t out_dtype, float* lse, void* stream);

/*
 * Decode attention with run-time termination (ART page, sections 2.1-2.4).  One new query
 * token per sequence and query head attends to the sequence's K/V cache (keys 0 .. seqlen-1)
 * block by block, block 0 first, then the other blocks most recent first.  After each block
 * the partial output's probe vector (its first 16 coordinates) is compared with the previous
 * one; once the change of its L2 norm stays below tau and its change of direction
 * (1 - cosine similarity) below phi for `patience` consecutive blocks, the traversal stops
 * and the partial output (over the blocks seen) is the result.  patience = 0 never stops.
 *   p            batch = sequences, seqlen = cached tokens, block = tile = 64 (the block the
 *                rule works on), n_q_heads / n_kv_heads <= 4, dtype SA_BF16; score_mode and
 *                output_aware are not used.
 *   Q            [B, Hq, d] in p->dtype: the decode tokens.
 *   K, V         [B, seqlen, Hkv, d] in p->dtype (the cache, BSHD as elsewhere).
 *   tau, phi     finite, >= 0;  patience >= 0.
 *   O            [B, Hq, d] in out_dtype, written.
 *   blocks_done  int32 [B, Hq], written: blocks each head processed (seqlen / 64 if it never
 *                stopped).
 * The stop decision is taken in fp32; near a threshold it may differ from one taken in exact
 * arithmetic.
 */
int sparse_attn_decode_art(const sa_problem* p, const void* Q, const void* K, const void* V,
                           float softmax_scale, float tau, float phi, int32_t patience, void* O,
                           int32_t out_dtype, int32_t* blocks_done, void* stream);

/*
 * sparse_attn_select without a caller workspace, for callers that cannot allocate device
 * memory (code under stream capture into a graph, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, results and validation as sparse_attn_select minus ws and
 * ws_bytes: the workspace is a 64 MiB array inside the library, one per GPU, held until the
 * process ends.  Problems whose sparse_attn_select_workspace_bytes exceeds 64 MiB
 * (67108864 bytes) are refused with SA_ERR_UNSUPPORTED before any HIP call.  Nothing is
 * allocated or freed.  Every call on one GPU shares that GPU's array: calls that overlap in
 * time on one GPU (concurrent streams, or threads) race and must be ordered by the caller.
 * Nothing in the array needs to start at zero (each call writes what it reads).
 */
int sparse_attn_select_noalloc(const sa_problem* p, const sa_budget* b, const void* Q,
                               const void* summaries, int32_t* kv_idx, int32_t* kv_cnt,
                               float* sigma, float* sigma_bar, uint8_t* gate, float* tau,
                               void* stream);

/* The calling thread's last error message ("" if none).  Valid until its next call. */
const char* sparse_attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H_ */
