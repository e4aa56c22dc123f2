/*
 * lmtopk.h - C ABI of liblmtopk: the LM-head (vocabulary) projection fused with
 * exact top-k selection, for AMD Instinct MI355X (gfx950).
 *
 * What is computed (lm-head-topk page, intro and section "Method"): for every
 * decode row m the library forms the logits L[m, v] of all V vocabulary entries
 * and returns only the k largest, as (values [M,k] fp32, indices [M,k] int64)
 * sorted by value descending; equal values are ordered by the lower vocabulary
 * index first (section "Method", last sentence; section "API").  The full logit
 * vector is never written to device memory: each chunk of the vocabulary is
 * scored on chip and offers its own exact top-k, and a merge pass reduces the
 * chunk candidates (section "Method").
 *
 * Conventions shared by every entry point
 *  - All array arguments are DEVICE pointers unless stated otherwise; `stream`
 *    is a hipStream_t passed as void* (NULL = the null stream).
 *  - Every call is asynchronous on `stream`.  The library allocates and frees
 *    no memory; the caller owns every buffer, including outputs and workspace.
 *    Inputs are read only; outputs are fully overwritten on success.
 *  - Arrays are dense and row-major.  Every pointer must be 16-byte aligned.
 *  - Arguments are checked on the host BEFORE anything is enqueued.  The only
 *    HIP calls made before that are read-only queries of the current device
 *    (its LDS limit per workgroup).  On any error status nothing is launched
 *    and nothing is written.  A failure reported by the HIP runtime while
 *    enqueueing maps to LMTOPK_ERR_HIP; a fault inside a kernel surfaces at
 *    the caller's next synchronisation, as for any asynchronous HIP work.
 *  - The library keeps no state of its own and is thread safe.  The caller's
 *    workspace carries its first 65,792 bytes from call to call: a
 *    completion counter (256 bytes) and eight per-row key histograms (8 KiB
 *    each), which must be zero before a call starts.  Prepare a new
 *    workspace once with lmtopk_workspace_init (or any zero fill); every call
 *    leaves them zero again when it completes and overwrites whatever else it
 *    reads.  Calls that share a workspace must be ordered on
 *    one stream; calls that overlap in time need workspaces of their own.
 *  - Inputs must be finite or +-inf.  NaN anywhere is outside the contract and
 *    gives an unspecified (but memory-safe) result.
 *  - +0.0 and -0.0 compare equal: they tie and the lower index comes first.
 *    A returned value keeps the bits of that index's own logit.
 *
 * Limits (lm-head-topk page, section "Requirements and limits"): 1 <= k <=
 * min(V, 2048).  Rows per call: 1 <= M <= 8 (the page tests 1 to 8 rows in its
 * section "Correctness"); every weight byte is read once per call for all M
 * rows.  V < 2^31.
 */
#ifndef LMTOPK_H
#define LMTOPK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------------ */
/* Status codes                                                              */
/* ------------------------------------------------------------------------ */
typedef enum {
  LMTOPK_OK = 0,
  LMTOPK_ERR_NULL = 1,      /* a required pointer is NULL                     */
  LMTOPK_ERR_SHAPE = 2,     /* M not in [1,8], V < 1, V >= 2^31, H < 1, ld < V,
                               or a size limit below is exceeded              */
  LMTOPK_ERR_K = 3,         /* k < 1 or k > min(V, 2048)                      */
  LMTOPK_ERR_GROUP = 4,     /* group_size != 128 or H % 128 != 0 (binary)     */
  LMTOPK_ERR_DTYPE = 5,     /* unknown lmtopk_dtype                           */
  LMTOPK_ERR_ALIGN = 6,     /* a pointer is not 16-byte aligned, or a dense
                               row is not a whole number of 16-byte vectors   */
  LMTOPK_ERR_WORKSPACE = 7, /* workspace NULL or smaller than required        */
  LMTOPK_ERR_OPTIONS = 8,   /* invalid lmtopk_options field                  */
  LMTOPK_ERR_HIP = 9        /* the HIP runtime refused a launch               */
} lmtopk_status;

typedef enum { LMTOPK_F32 = 0, LMTOPK_BF16 = 1 } lmtopk_dtype;

/* Optional per-call settings; pass NULL for the defaults. */
typedef struct {
  /* Vocabulary rows per chunk (one workgroup scores and selects one chunk).
     0 = automatic.  Otherwise a multiple of 64 that is <= 1024, or 2048
     (lmtopk_binary: 2048 only for M <= 2, OPTIONS otherwise).  The result
     never depends on this value. */
  int32_t chunk_rows;
  int32_t reserved; /* must be 0 */
  /* If not NULL: the address of two hipEvent_t (an array void*[2]).  The
     chunk-scoring kernel is then launched with hipExtLaunchKernel so that the
     first event records the kernel's start and the second its end, which
     times that kernel apart from the merge kernels after it.  The events
     must exist; the library does not own them. */
  void* score_events;
  /* If not NULL: a device array of M floats that receives, for each row,
     the log-sum-exp of all V of its logits, log(sum_v exp(L[m, v])), so
     that values[m, i] - lse[m] are the top-k log-probabilities (Selective
     Log Softmax page, section "Kernel design", online log-sum-exp: per
     slice a maximum and a sum of exponentials, then combined).  Each chunk
     reduces its rows to one (max, sum) pair (its waves' pairs combined in
     LDS) and the final merge combines the chunks' pairs; no weight byte is
     read twice.  An +inf logit gives +inf;
     a row whose logits are all -inf gives -inf.  16-byte aligned. */
  float* lse;
  /* If not NULL: a device bitmask [M][ceil(V / 32)] of int32 words; bit
     (v % 32) of word v / 32 of row m is 1 if vocabulary entry v is allowed
     (logits-processor page, section "API": a grammar's bitmask, bit 1 =
     allowed, disallowed logits set to -inf).  A disallowed entry's logit
     counts as -inf, for the top-k and for lse alike: it is returned only
     when fewer than k entries are allowed, after every allowed one, in index
     order.  Bits past V are ignored.  16-byte aligned. */
  const int32_t* allowed;
  /* If not NULL: draw one token per row from the call's top-k survivors
     (lmtopk_sampling below).  A host pointer, read during the call. */
  const struct lmtopk_sampling* sampling;
} lmtopk_options;

/*
 * Sampling one token per row from the top-k survivors (logits-processor
 * page, section "API": sample(logits, temperature, top_k, top_p, min_p,
 * seed, offset); section "Method": the three filters meet in one keep set
 * and the token is drawn by Gumbel-max over it).  The draw is fused after
 * the exact top-k, so it sees the call's k survivors in output order
 * (value descending, lower index first) and never a token outside them.
 * For row m, with T its temperature, z_i = values[m, i] * (1 / T) in fp32
 * and lse_T = log sum over all V entries of exp(L[m, v] / T) (the whole
 * vocabulary; disallowed entries of a bitmask count as -inf):
 *   - the keep set is a prefix of the survivors: position 0 always; position
 *     i >= 1 while every earlier one was kept and
 *       i < top_k                       (top_k <= 0 or >= k: any i < k),
 *       p_0 + ... + p_{i-1} < top_p,   p_j = exp(z_j - lse_T)   (top_p < 1),
 *       exp(z_i - z_0) >= min_p                                 (min_p > 0),
 *       z_i > -inf;
 *   - the token is the index of the kept position with the largest
 *     z_i + g_i, g_i = -log(-log(u_i)), the lower position on a tie; u_i is
 *     the uniform of Philox4x32-10 (Salmon et al., SC 2011) at key (seed mod
 *     2^32, seed div 2^32) and counter (vocabulary index, m, offset mod 2^32,
 *     offset div 2^32): its first output word x, u = (x >> 9) * 2^-23 +
 *     2^-24;
 *   - temperature <= 0 is greedy: the token is indices[m, 0] (the argmax,
 *     lower index on ties), keep-set size 1; likewise when values[m, 0] is
 *     +inf or every logit of the row is -inf.
 * With sampling, lmtopk_options.lse (if given) receives lse_T, the
 * normaliser of the distribution sampled from (log-sum-exp of L / T; of L
 * itself for greedy rows).  Each parameter applies to every row unless its
 * per-row device array is given.  Cost: the survivors' k values are already
 * on chip; top-p (any row with top_p < 1, or top_p_rows given) adds the
 * per-chunk normaliser partials of the lse option.
 */
typedef struct lmtopk_sampling {
  float temperature;               /* <= 0: greedy                          */
  int32_t top_k;                   /* <= 0: off; must be <= k (else OPTIONS) */
  float top_p;                     /* >= 1: off                             */
  float min_p;                     /* <= 0: off                             */
  const float* temperature_rows;   /* [M] device, or NULL                   */
  const int32_t* top_k_rows;       /* [M] device, or NULL (a value above k
                                      or <= 0 means k)                      */
  const float* top_p_rows;         /* [M] device, or NULL                   */
  const float* min_p_rows;         /* [M] device, or NULL                   */
  uint64_t seed;
  uint64_t offset;                 /* advance it every decoding step        */
  const uint64_t* offset_device;   /* [1] device, or NULL: if given, the
                                      offset is read from it when the call
                                      runs (a captured graph can then be
                                      replayed with a new offset)           */
  int64_t* tokens;                 /* out [M] device                        */
  int32_t* kept;                   /* out [M] device, or NULL: keep-set size */
} lmtopk_sampling;

/* ------------------------------------------------------------------------ */
/* Packed binary head, layout version 1                                      */
/* ------------------------------------------------------------------------ */
/*
 * A binary head stores each weight as a sign (+1 or -1) and each group of 128
 * consecutive weights of one vocabulary row as one fp32 scale, so that the
 * dequantized weight is sign * scale (lm-head-topk page, section "Usage" for
 * the argument list and group_size=128; section "Requirements and limits" for
 * packing as a separate offline step).  The pages do not give the packed
 * layout; this library defines its own:
 *
 *   G   = H / 128             groups per vocabulary row
 *   G4  = ceil(G / 4) * 4     groups rounded up to whole quads
 *   V64 = ceil(V / 64) * 64   vocabulary rows rounded up to whole 64-row tiles
 *   row v lives in tile t = v / 64 at lane r = v % 64
 *
 *   wq     : uint32 words, word index ((t * G + g) * 64 + r) * 4 + w for
 *            g < G, w < 4.  Bit b (value 1 << b) of that word is the sign of
 *            element j = 128 * g + 32 * w + b of row v: 1 means +1 (the
 *            source weight was >= 0, so -0.0 packs as +1), 0 means -1.
 *            Size V64 * H / 8 bytes.
 *   wscale : fp32, index ((t * (G4 / 4) + q) * 64 + r) * 4 + i holds the
 *            scale of group g = 4 * q + i of row v.  Size V64 * G4 * 4 bytes.
 *
 *   Rows v >= V and groups g >= G are padding: their sign words and scales
 *   are 0.  The scoring kernels never offer padding rows as candidates.
 *
 * One 64-lane wavefront reading one uint4 per lane (one group of one row per
 * lane) thus reads 1 KiB of contiguous memory, and one float4 per lane reads
 * the scales of four consecutive groups.
 */
#define LMTOPK_LAYOUT_VERSION 1
#define LMTOPK_GROUP_SIZE 128
#define LMTOPK_MAX_ROWS 8
#define LMTOPK_MAX_K 2048
/* Binary path: the activation bit planes of all M rows live in LDS
   (132 bytes per row and group of 128, about 1.03 * M * H bytes). */
#define LMTOPK_MAX_BINARY_MH 65536

/* Layout version of packed heads this library reads and writes. */
int32_t lmtopk_layout_version(void);

/* Human-readable name of a status code (static storage; never NULL). */
const char* lmtopk_status_string(lmtopk_status s);

/* Host-only: byte sizes of the two packed arrays for a V x H head.
   Errors: NULL (an out pointer), SHAPE (V < 1, V >= 2^31, H < 1),
   GROUP (group_size != 128 or H % 128 != 0). */
lmtopk_status lmtopk_packed_bytes(int64_t V, int64_t H, int32_t group_size,
                                  size_t* wq_bytes, size_t* wscale_bytes);

/* Host-only: workspace bytes needed by lmtopk_binary, lmtopk_dense and
   lmtopk_select for these sizes and options.  The same workspace serves all
   three.  It holds a 256-byte completion counter (zero between calls: the
   workgroup that finishes a chunk launch last merges the candidates itself
   when they fit it and k <= 256, instead of a second launch) and eight
   2,048-bin key histograms of 8 KiB (zero between calls: a merge with an
   intermediate level counts the candidates' keys there, by their top 11
   bits, and its first level keeps only those in or above the bin of the
   row's k-th largest), then, per row and chunk,
   the chunk's four best candidates and all its candidates (8 bytes each),
   plus one intermediate merge level when a row has more than 16384
   candidates, plus 8 bytes per row and chunk for the log-sum-exp pairs.
   Errors: NULL, SHAPE, K, OPTIONS. */
lmtopk_status lmtopk_workspace_bytes(int64_t M, int64_t V, int32_t k,
                                     const lmtopk_options* opt, size_t* bytes);

/* Host-only: the chunking lmtopk_binary uses for these sizes and options:
   vocabulary rows per chunk (one workgroup scores and selects one chunk),
   the number of chunks, and the waves of a chunk workgroup.  With
   chunk_rows 0 the library takes 1,024-row chunks, or, when at most 128 of
   them would cover V (leaving CUs idle) and the final merge can still run in
   the chunk launch, 512-row chunks scored by two waves per 64-row tile (one
   per half of the groups; also for any chunk of up to 512 rows where the
   LDS allows).  The values never change a result.
   Errors: NULL, SHAPE, K, GROUP, OPTIONS. */
lmtopk_status lmtopk_binary_plan(int64_t M, int64_t V, int64_t H, int32_t k,
                                 const lmtopk_options* opt, int32_t* chunk_rows,
                                 int32_t* n_chunks, int32_t* waves);

/* Zero-fill a workspace of `bytes` bytes (device pointer, 16-byte aligned)
   on `stream`, with a kernel rather than a memset so that the call may be
   captured into a graph.  Needed once per new workspace (see the
   conventions above); calls leave it ready for the next call.
   Errors: NULL, ALIGN, HIP. */
lmtopk_status lmtopk_workspace_init(void* workspace, size_t bytes, void* stream);

/*
 * Pack a dense head into the layout above (offline; once per model).
 *   w      : [V, H] row-major, fp32 or bf16 (w_dtype).
 *   wq     : out, lmtopk_packed_bytes(...).wq_bytes bytes.
 *   wscale : out, lmtopk_packed_bytes(...).wscale_bytes bytes.
 * Sign: +1 iff w >= 0.  Scale of a group: the mean of |w| over its 128
 * elements, summed in fp64 and rounded once to fp32.
 * Errors: NULL, SHAPE, GROUP, DTYPE, ALIGN, HIP.
 */
lmtopk_status lmtopk_pack_binary(const void* w, lmtopk_dtype w_dtype, int64_t V,
                                 int64_t H, int32_t group_size, void* wq,
                                 float* wscale, void* stream);

/*
 * Binary head: logits, then exact top-k (lm-head-topk page, section "Usage",
 * binary entry point; section "Correctness" for what it must match).
 *   act_q     : [M, H] int8 activations (the full int8 range is accepted).
 *   act_scale : [M] fp32 per-row activation scale.
 *   wq, wscale: packed head (layout above) of V rows and H columns.
 *   bias      : [V] fp32 or NULL.
 *   values    : out [M, k] fp32;  indices : out [M, k] int64.
 *   workspace : lmtopk_workspace_bytes(M, V, k, opt) bytes, device.
 * Logit of row m, entry v (G = H / 128 groups, Q = ceil(G / 4) quads of
 * groups, Gh = 4 * floor(Q / 2)):
 *   D_g = sum over the 128 j of group g of act_q[m, j] * sign[v, j]  (exact)
 *   lo  = fp32 fused multiply-add chain over g = 0, 1, ..., Gh-1 of
 *         (float)D_g * wscale[v, g], starting from 0
 *   hi  = the same chain over g = Gh, ..., G-1, starting from 0
 *   L   = fmaf(lo + hi, act_scale[m], bias ? bias[v] : 0)
 * (the same operations for every chunk size, M and option, so a row's
 * logits never depend on them)
 * Errors: NULL, SHAPE (also M * H > LMTOPK_MAX_BINARY_MH), K, GROUP, ALIGN,
 * WORKSPACE, OPTIONS (also chunk_rows 2048 with M > 2), HIP.
 */
lmtopk_status lmtopk_binary(const int8_t* act_q, const float* act_scale,
                            const void* wq, const float* wscale,
                            const float* bias, int64_t M, int64_t V, int64_t H,
                            int32_t group_size, int32_t k, float* values,
                            int64_t* indices, void* workspace,
                            size_t workspace_bytes, const lmtopk_options* opt,
                            void* stream);

/*
 * Dense head: logits, then exact top-k (lm-head-topk page, section "Usage",
 * dense entry point, which the page keeps as the correctness reference).
 *   hidden : [M, H], weight : [V, H]; both fp32 or both bf16 (dtype).
 *   bias   : [V] fp32 or NULL.
 * L[m, v] = sum_j hidden[m, j] * weight[v, j] accumulated in fp32 (products of
 * bf16 inputs are exact in fp32) in one fixed order that is the same for every
 * (m, v), then + bias[v].
 * H * element size must be a multiple of 16 bytes (ALIGN otherwise).
 * Errors: NULL, SHAPE, K, DTYPE, ALIGN, WORKSPACE, OPTIONS, HIP.
 */
lmtopk_status lmtopk_dense(const void* hidden, const void* weight,
                           lmtopk_dtype dtype, const float* bias, int64_t M,
                           int64_t V, int64_t H, int32_t k, float* values,
                           int64_t* indices, void* workspace,
                           size_t workspace_bytes, const lmtopk_options* opt,
                           void* stream);

/*
 * Selection stage alone on logits already in device memory: the exact top-k
 * of logits[m, 0:V] for each row (row stride ld >= V elements).  This is the
 * lm-head-topk page's second half on its own (section "Method": each chunk
 * offers its top-k, a merge reduces them), applied to materialized logits,
 * the form its section "Correctness" compares against (torch.topk on the
 * materialized logits).  Same chunked select and merge kernels as the fused
 * paths, so the chunk select and merge can be checked bit for bit against a
 * plain sort; with lmtopk_options.sampling it is also the logits-processor
 * page's sample() restricted to the top-k.
 * Errors: NULL, SHAPE, K, ALIGN, WORKSPACE, OPTIONS, HIP.
 */
lmtopk_status lmtopk_select(const float* logits, int64_t M, int64_t V,
                            int64_t ld, int32_t k, float* values,
                            int64_t* indices, void* workspace,
                            size_t workspace_bytes, const lmtopk_options* opt,
                            void* stream);

/*
 * lmtopk_binary without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, checks, kernels and
 * results as lmtopk_binary; its workspace is a device array inside the
 * library, LMTOPK_NOALLOC_SCRATCH_BYTES bytes per GPU, held from its first
 * use on a GPU until the process ends.  The call itself allocates nothing.
 * Calls on one GPU share that array: calls that overlap in time on one GPU
 * (several streams or threads at once) race and give wrong results; order
 * them.  The first call on a GPU also enqueues one small fill kernel on
 * `stream` that clears the array's completion counter and key histograms.
 * Errors: as lmtopk_binary; WORKSPACE when lmtopk_workspace_bytes for these
 * sizes and options exceeds LMTOPK_NOALLOC_SCRATCH_BYTES.
 */
#define LMTOPK_NOALLOC_SCRATCH_BYTES (8u << 20)
lmtopk_status lmtopk_binary_noalloc(const int8_t* act_q, const float* act_scale,
                                    const void* wq, const float* wscale,
                                    const float* bias, int64_t M, int64_t V,
                                    int64_t H, int32_t group_size, int32_t k,
                                    float* values, int64_t* indices,
                                    const lmtopk_options* opt, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LMTOPK_H */
