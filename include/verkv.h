/* verkv.h - C ABI of the VerKV decode path (PoissonComp at prefill, KVFetch at
 * decode) for AMD Instinct MI355X (gfx950).
 *
 * Method: "Verify Before You Fetch: Reliable KV Cache Compression for LLM
 * Inference" (arXiv 2611.11319).  The picx.dev summary page, section
 * "Methodology", defines every operation named below: PoissonComp (eq. 3 and the
 * Poisson sample), the bounded shrinkage estimator (Definition 2, eq. 5), the
 * Bernstein certificate (Lemma 1, eq. 7) and KVFetch steps 1-5 (eqs. 9-10).  The
 * paperdot.bitmofang.com abstract page states the setting: pivotal tokens and a
 * token-level sketch resident on the GPU, the complete cache in CPU memory, and a
 * user-specified (eps, delta) tolerance.
 *
 * Conventions for every entry point
 *  - Pointers are device pointers unless marked [host] or [pinned host].  Pinned
 *    host buffers must come from hipHostMalloc (or an allocator built on it); the
 *    kernels read them directly over the host link.
 *  - Every buffer is owned by the caller; the library allocates no device or
 *    host memory in these calls.  Work is enqueued on `stream` (0 = the null
 *    stream) and the calls return before it completes, except verkv_compress,
 *    which synchronises `stream` once to read the pivot counts.
 *  - Errors are returned as verkv_status; nothing else crosses the ABI.
 *    Argument errors are detected on the host before any work is enqueued.  A
 *    HIP runtime error maps to VERKV_EHIP (the message is kept per thread, see
 *    verkv_last_error).
 *  - head_dim must be 128.  GQA group G = (query heads)/(KV heads) in 1..8.
 *
 * Layouts (sequence-major, ragged batches of B sequences with lengths n_b and token
 * capacities c_b >= n_b, c_b = n_b unless verkv_shape.seq_cap is given; a sequence's
 * per-head arrays are strided by c_b so that verkv_append can grow it in place):
 *  - token arrays      [B][Hkv][c_b]           sequence b starts at Hkv * sum_{b'<b} c_b'
 *  - bit arrays        [B][Hkv][ceil(c_b/32)]  token i is bit (i % 32) of word i / 32
 *  - cache rows        [B][Hkv][c_b][128]      kv_dtype elements; tokens i < n_b are used
 *  - query rows        [B][Hq][128] float32    Hq = Hkv * G; row h uses KV head h / G
 *  - per-row outputs   [B][Hq]
 *  - pivot ids         [B][Hkv][cap]
 *  - pivot K/V rows    [verkv_pivot_rows(s, cap)][128], in the order the pivot-attention
 *                      kernel reads them (written by verkv_compress; opaque to callers)
 */
#ifndef VERKV_H
#define VERKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *verkv_stream_t;   /* the same object as hipStream_t */

typedef enum {
  VERKV_OK = 0,
  VERKV_EINVAL = -1,        /* bad argument (range, null pointer, tau outside [0,1]) */
  VERKV_EBUDGET = -2,       /* eta * n_b is below the sink + local token count        */
  VERKV_ECAPACITY = -3,     /* a pivot set does not fit `cap`; *needed_cap is set     */
  VERKV_EHIP = -4,          /* HIP runtime error                                       */
  VERKV_EUNSUPPORTED = -5,  /* head_dim != 128, G > 8, too many sequences or tokens   */
  VERKV_EWORKSPACE = -6     /* workspace smaller than the size helper returned        */
} verkv_status;

typedef enum { VERKV_BF16 = 0, VERKV_F32 = 1 } verkv_dtype;

#define VERKV_HEAD_DIM 128
#define VERKV_MAX_GROUP 8
#define VERKV_MAX_BATCH 128
#define VERKV_MAX_SEQ_LEN (1 << 20)

/* Shape of one layer of a batch. */
typedef struct {
  int32_t batch;            /* B, 1..VERKV_MAX_BATCH                                   */
  int32_t n_kv_heads;       /* Hkv >= 1                                                */
  int32_t group;            /* G = Hq / Hkv, 1..VERKV_MAX_GROUP                        */
  int32_t head_dim;         /* must be 128                                             */
  const int32_t *seq_len;   /* [host][B], each 1..VERKV_MAX_SEQ_LEN                    */
  int32_t n_sink;           /* first n_sink tokens are always kept (H)                 */
  int32_t n_local;          /* last n_local tokens are always kept (H)                 */
  int32_t kv_dtype;         /* verkv_dtype of the cache, the pivots and the sketch     */
  uint32_t layer;           /* third Philox counter word                               */
  const int32_t *seq_cap;   /* [host][B] token capacity c_b >= n_b of each sequence's  */
                            /* arrays, each <= VERKV_MAX_SEQ_LEN (NULL: c_b = n_b)      */
  int32_t stage_slots;      /* host rows per KV head the cross-step staging holds (see */
                            /* verkv_state.v_host); 0: min(8192, 65536 / (B Hkv), the   */
                            /* limit below).  When key rows are staged beside the       */
                            /* values (sketch_exact 0) a slot takes two rows, so half   */
                            /* as many tokens are staged.  At most 2^(32 - t) - 1 where  */
                            /* t is the bits of the largest capacity (a host-row list   */
                            /* entry packs the token and its slot + 1 into 32 bits):    */
                            /* 131071 at 32K tokens, 4095 at 2^20 (VERKV_EINVAL beyond, */
                            /* checked with the shape).  The decode workspace grows by  */
                            /* about (row bytes + 12 B) x B x Hkv per slot.             */
} verkv_shape;

/* GPU-resident compressed state of one layer (written by verkv_compress; the decode
 * calls read it as written there, so a state that no verkv_compress call of the same
 * shape and capacity filled gives meaningless results). */
typedef struct {
  double *r;                /* [B][Hkv][n_b] inclusion probability, 1 on H             */
  uint32_t *resident;       /* [B][Hkv][ceil(n_b/32)] bit set for tokens of H u S      */
  int32_t *piv_idx;         /* [B][Hkv][cap] ascending token ids of H u S              */
  int32_t *piv_count;       /* [B][Hkv] |H u S|                                        */
  void *piv_k;              /* [verkv_pivot_rows(s, cap)][128] kv_dtype: keys of H u S  */
  void *piv_v;              /* same for the values; row order set by verkv_compress    */
  int32_t cap;              /* pivot capacity per (sequence, KV head)                  */
  const void *sketch;       /* [B][Hkv][n_b][128] kv_dtype token-level key sketch      */
                            /* (or 2-bit rows, see sketch_format), on the device.      */
                            /* Exact-sketch mode: the keys themselves.                 */
  int32_t sketch_exact;     /* 1: the sketch rows are the keys, so the host fetch of    */
                            /* KVFetch step 5 reads only the value rows and takes the  */
                            /* weights w_i = w_hat_i of step 1; 0: it reads K and V.   */
  const void *v_host;       /* [pinned host][B][Hkv][n_b][128] kv_dtype: the value     */
                            /* cache verkv_refine reads (may be NULL).  With it (and,   */
                            /* when sketch_exact is 0, with k_host as well), the steps  */
                            /* on one workspace keep host rows staged in it: the rows   */
                            /* of the first stage_slots entries of a step's host-row    */
                            /* list, planned at the end of verkv_refine and read from   */
                            /* v_host by the next verkv_decode_step while its decision  */
                            /* kernel runs (a row staged already stays where it is);    */
                            /* verkv_refine then takes the rows it needs from there.    */
                            /* Staged rows are reused only for the same v_host address  */
                            /* and array layout (capacities), so the rows of v_host     */
                            /* must not change between the steps that share a           */
                            /* workspace (rows appended by verkv_append are new rows).  */
                            /* Results do not depend on it.                             */
  int32_t sketch_format;    /* VERKV_SKETCH_ROWS (0): `sketch` holds kv_dtype rows as   */
                            /* above; VERKV_SKETCH_2BIT (1): `sketch` holds 64-byte     */
                            /* rows written by verkv_quantize_sketch (needs            */
                            /* sketch_exact = 0: fetched rows are scored from the host */
                            /* keys).                                                   */
  double *level;            /* [B][Hkv] written by verkv_compress (may be NULL): the    */
                            /* water level c of eq. 3, or the branch that set r on the */
                            /* non-forced tokens (-1 all in H, -2 no budget left, -3   */
                            /* every positive score saturated); verkv_append needs it. */
  const void *k_host;       /* [pinned host][B][Hkv][n_b][128] kv_dtype: the key cache  */
                            /* (may be NULL).  When sketch_exact is 0 the host fetch   */
                            /* reads key rows too; with k_host and v_host both set,     */
                            /* the staging keeps each row's key beside its value        */
                            /* (same rules as v_host above; staged rows are reused only */
                            /* for the same pair of caches).  Ignored when sketch_exact */
                            /* is 1.  Without it a non-exact sketch stages nothing.     */
} verkv_state;

#define VERKV_SKETCH_ROWS 0
#define VERKV_SKETCH_2BIT 1
#define VERKV_SKETCH2_ROW_BYTES 64

/* The 2-bit key sketch (the pages evaluate one but give no quantiser; this one is
 * asymmetric uniform quantisation per token row in groups of 32 dimensions): for each
 * group, mn = min, sc = (max - min) / 3 in float32, code_j = the number of midpoints
 * mn + (c + 1/2) sc, c = 0, 1, 2, that x_j reaches (float64), and the sketch key is
 * x_hat_j = mn + code_j sc (float64).  Row layout, 64 bytes per (sequence, KV head,
 * token): bytes 0-31 eight 32-bit words, word w holding the codes of dimensions
 * 8w..8w+7 in bits 0-15 and of 8(w+8)..8(w+8)+7 in bits 16-31, two bits per dimension
 * in order; bytes 32-63 eight float32: mn, sc of groups 0, 2, 1, 3.
 *   K       [B][Hkv][n_b][128] kv_dtype key cache, device memory or pinned host memory
 *   sketch  [B][Hkv][n_b][64] bytes (device), written
 * Asynchronous on `stream`. */
verkv_status verkv_quantize_sketch(const verkv_shape *s, const void *K, void *sketch,
                                   verkv_stream_t stream);

/* Per-step results.  Row arrays are [B][Hq]; KV-head arrays are [B][Hkv]. */
typedef struct {
  /* written by verkv_decode_step */
  double *m_hat;            /* largest sketch score q.k/sqrt(d) (the softmax shift)     */
  double *d_sketch;         /* D = sum over all n_b tokens of exp(s_hat - m_hat)       */
  double *beta_star;        /* self-consistent shrinkage bias (Definition 2)           */
  double *eps_hat;          /* eps_hat(L) of eq. 7                                     */
  uint8_t *certified;       /* 1 when eps_hat(L) < eps (no fetch for this row)          */
  int32_t *kstar;           /* k* of eq. 10 (0 when certified)                         */
  int32_t *fetch_idx;       /* [B][Hkv][fetch_cap] ascending union F over the group    */
                            /* (may be NULL; lists longer than fetch_cap are cut)       */
  int32_t fetch_cap;
  int32_t *fetch_count;     /* |F| per KV head                                         */
  int32_t *h2d_count;       /* |F \ S|: rows read from host memory per KV head         */
  /* written by verkv_refine */
  double *eps_after;        /* eps_hat(L \ F) with lambda frozen                       */
  float *n_hat;             /* [B][Hq][128] N_hat (shifted by m_hat)                   */
  float *d_hat;             /* D_hat (shifted by m_hat)                                */
  float *o;                 /* [B][Hq][128] attention output N_hat / D_hat             */
  float *lse;               /* m_hat + ln D_hat                                        */
} verkv_step_out;

/* PoissonComp (prefill), per (sequence b, KV head g): r_i = min(1, c tau_i) water-
 * filled so that sum_i r_i = eta * n_b with the first n_sink and last n_local tokens
 * forced to r = 1 (picx.dev summary, "POISSONCOMP", eq. 3); then Z_i ~ Bernoulli(r_i)
 * from Philox4x32-10 with counter (i, g, layer, b) and key (seed mod 2^32, seed >> 32);
 * H u S compacted in ascending order and their K/V rows copied from the pinned host
 * cache into piv_k / piv_v.
 *   tau       [B][Hkv][n_b] float32 importance scores in [0, 1] (device)
 *   K_host,   [pinned host][B][Hkv][n_b][128] kv_dtype complete cache
 *   V_host
 *   eta       resident fraction, 0 < eta <= 1
 *   workspace at least verkv_compress_workspace_bytes(s)
 *   needed_cap [host, may be NULL] on VERKV_ECAPACITY: the largest |H u S|
 * Returns VERKV_EBUDGET if fl(eta * n_b) < min(n_b, n_sink + n_local) for some b,
 * VERKV_EINVAL if some tau is outside [0, 1] (detected on the device; state is then
 * undefined).  Synchronises `stream` once. */
verkv_status verkv_compress(const verkv_shape *s, const float *tau, const void *K_host,
                            const void *V_host, double eta, uint64_t seed, verkv_state *st,
                            void *workspace, size_t workspace_bytes, int32_t *needed_cap,
                            verkv_stream_t stream);
size_t verkv_compress_workspace_bytes(const verkv_shape *s);

/* A growing cache: token n_b is appended to every sequence b of the batch (the pages
 * compress the cache once, at prefill, and are silent on decode-time growth; this is
 * the reading taken, with the prefill's rule of the picx.dev summary page, "POISSONCOMP",
 * eq. 3).  The new token joins the local window (r = 1, resident).  The token leaving
 * the window, t = n_b - n_local (none when t < n_sink), gets the prefill's rule with the
 * water level verkv_compress recorded in st->level: r_t = min(1, c ceil(tau_t 2^40))
 * (1 / 0 / [tau_t > 0] for the other branches), and when 0 < r_t < 1 its Bernoulli draw
 * from the Philox counter (t, g, layer, b) it would have had at prefill; it stays a
 * pivot only if drawn.  With n_local = 0 the new token itself takes the rule.  The
 * level is not re-solved.  r, the resident bits, the ascending pivot list, its count
 * and the pivot K/V rows (re-laid out in the order the pivot attention reads them) are
 * updated in place.
 *   s       the shape BEFORE the append (lengths n_b); every n_b + 1 <= c_b
 *   tau     [B][Hkv][c_b] scores; the caller has written the new token's at index n_b
 *   K_host, [pinned host][B][Hkv][c_b][128] the cache, with the new token's rows written
 *   V_host  at row n_b (the caller also writes its key into an exact sketch)
 *   seed    the seed verkv_compress drew with
 *   status  [device] 4 bytes: cleared, then the kernels OR 1 (a score outside [0, 1]),
 *           8 (a pivot list would exceed st->cap), 16 (the state does not match the
 *           shape); with any of them set nothing was changed
 *   workspace at least verkv_append_workspace_bytes(s, st->cap)
 * Asynchronous on `stream`; afterwards the caller's shape has lengths n_b + 1.  A 2-bit
 * sketch must be re-quantised by the caller for the new rows. */
verkv_status verkv_append(const verkv_shape *s, verkv_state *st, const float *tau,
                          const void *K_host, const void *V_host, uint64_t seed, int32_t *status,
                          void *workspace, size_t workspace_bytes, verkv_stream_t stream);
size_t verkv_append_workspace_bytes(const verkv_shape *s, int32_t cap);

/* Rows of 128 kv_dtype elements that st->piv_k and st->piv_v must each hold for pivot
 * capacity `cap` (0 for an invalid shape or cap < 1).  verkv_compress stores the pivot
 * rows in the order in which the resident-pivot attention's persistent workers read
 * them: the pivots of all KV heads, head after head, cut into 32-row chunks and shared
 * evenly among the workers, worker w's i-th chunk at block i * P + w (P workers), so
 * the workers read one moving window of memory together.  The count is
 * (B * Hkv * ceil(cap / 32) + 768) * 32, a little more than B * Hkv * cap. */
size_t verkv_pivot_rows(const verkv_shape *s, int32_t cap);

/* KVFetch steps 1-4 (picx.dev summary, "KVFETCH"; Definition 2; Lemma 1): per query
 * row, sketch weights over all n_b tokens, the self-consistent shrinkage bias,
 * eps_hat(L), the certified flag, and when it fails the fetch order g (eq. 9) and k*
 * (eq. 10); per KV head the union F of the group's fetch sets, the fetch list and the
 * estimator coefficients of the resident pivots (1 on H u (S n F), lambda_i / r_i on
 * S \ F); per row the partial terms of eps_hat(L \ F) that verkv_refine finishes.
 *   q      [B][Hq][128] float32
 *   beta   multiplier kappa of the bias term inside the clip: 1 is the paper's
 *          estimator, +INFINITY gives lambda = 1 (Horvitz-Thompson), 0 gives
 *          lambda = r; must be >= 0
 *   eps    tolerance > 0;  delta  confidence parameter in (0, 1)
 *   workspace at least verkv_decode_workspace_bytes(s, st->cap); pass the same
 *          workspace to verkv_refine for this step.  Between steps it keeps each
 *          row's B*, which the next step on it takes as the starting point of its
 *          fixed-point search, the list of host rows the step read, and the staged
 *          rows with the plan verkv_refine made for the next step (see
 *          verkv_state.v_host).
 *          Results do not depend on these: zero-filled or foreign contents only cost
 *          time (staged rows carry the identity of the cache they came from).
 * No host synchronisation.  Host memory is read only by the staging copies (the rows
 * the previous step's plan asked for, see verkv_state.v_host).
 * out->o and out->lse are not written here: verkv_refine always follows, also when
 * every row is certified (then it finishes o from the resident-pivot partials and
 * reads nothing from the host).  The split is for overlap, not for skipping: the
 * resident-pivot attention runs beside the host reads inside verkv_refine, so a
 * step that finished certified rows here would put that attention on the critical
 * path of the rows that fetch.
 * One decode step per device at a time: the decision kernel groups the workgroups of
 * a query row into a team that exchanges partials through memory, and sizes the
 * teams so that every member is resident on the device at once.  Steps issued on
 * two streams of one device could leave members of each waiting for CUs the other
 * holds; the waits are bounded (status bit 4, verkv_check) but the step's results
 * are then wrong.  Serialise decode steps on one device (one stream, or events). */
verkv_status verkv_decode_step(const verkv_shape *s, const verkv_state *st, const float *q,
                               double beta, double eps, double delta, verkv_step_out *out,
                               void *workspace, size_t workspace_bytes, verkv_stream_t stream);

/* KVFetch step 5: attention partials over the resident pivots H u S, the rows F \ S
 * of V (and of K unless st->sketch_exact) read from the pinned host cache (zero-copy
 * loads issued by the kernels) with their exact terms, and the finished rows:
 * o = N_hat / D_hat, lse, n_hat, d_hat and eps_after = eps_hat(L \ F).
 * Must follow verkv_decode_step on the same stream with the same workspace, q, s
 * and st.  The resident-pivot attention runs on a second stream of the library (one
 * per device, default priority; verkv_decode_step put the pivot coefficients and the
 * eps_after terms there) while the host rows stream in on `stream`; the call joins
 * that stream back into `stream` before the finishing kernel, so every result is
 * ordered on `stream` as usual.  Rows whose KV head fetched nothing
 * are finished from the resident partials alone. */
verkv_status verkv_refine(const verkv_shape *s, const verkv_state *st, const float *q,
                          const void *K_host, const void *V_host, verkv_step_out *out,
                          void *workspace, size_t workspace_bytes, verkv_stream_t stream);
size_t verkv_decode_workspace_bytes(const verkv_shape *s, int32_t cap);
/* Of the rows F \ S the last verkv_refine on `workspace` needed (KVFetch step 5, picx.dev
 * summary page, "KVFETCH" step 5; out->h2d_count per KV head), how many it took from the
 * cross-step staging area instead of the host link, summed over the batch's KV heads
 * (*rows).  Each verkv_decode_step clears the count, and the host-row kernel adds to it.
 * The rest crossed the link.  workspace: the one the step used, of workspace_bytes
 * (at least verkv_decode_workspace_bytes(s, cap)).  Synchronises `stream`.  Errors:
 * VERKV_EINVAL (null pointers, cap < 1), VERKV_EWORKSPACE, a shape error as for a step. */
verkv_status verkv_staged_rows(void *workspace, size_t workspace_bytes, const verkv_shape *s,
                               int32_t cap, verkv_stream_t stream, int64_t *rows);

/* verkv_decode_step with options.  flags:
 *   VERKV_STEP_RESOLVED  the other reading of eqs. (9)-(10) (picx.dev summary page,
 *       "KVFETCH" steps 3-4): eq. (9) writes eps_hat(L \ {i}) without saying whether
 *       the shrinkage bias of Definition 2 follows the set.  verkv_decode_step keeps
 *       lambda frozen at its value for the full L; with this flag the order is still
 *       eq. (9)'s g (lambda frozen), but k* of eq. (10) is the least k for which
 *       eps_hat(L_g[k:]) with the bias solved on L_g[k:] alone is below eps, and the
 *       kept set L_g[k*:] keeps that bias (beta_star, the pivot coefficients and
 *       eps_after use it).  Certification (k* = 0) is the same test.  For beta = 0 or
 *       +INFINITY lambda does not depend on the bias: both readings make the same cut,
 *       and this one reports the kept set's bias sum(w (1 - lambda)) over L_g[k*:].
 * Other bits give VERKV_EINVAL.  verkv_refine follows as usual. */
#define VERKV_STEP_RESOLVED 1u
verkv_status verkv_decode_step_ex(const verkv_shape *s, const verkv_state *st, const float *q,
                                  double beta, double eps, double delta, verkv_step_out *out,
                                  void *workspace, size_t workspace_bytes, uint32_t flags,
                                  verkv_stream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): verkv_decode_step followed by
 * verkv_refine, same arguments and results, with the workspace in a static device array
 * of the library (verkv_noalloc_scratch_bytes() = 64 MiB, held on every device the
 * library runs on until the process ends) instead of a caller buffer.  Nothing is
 * allocated or created by the call; every kernel runs on `stream` (no second stream,
 * no cross-step staging of host rows, which only ever saves host-link reads).
 *   status  [device, may be NULL] the kernels OR their flags into it (4: a team
 *           barrier timed out, 2: a fixed point did not converge); the caller clears it
 * Returns VERKV_EWORKSPACE (with verkv_last_error naming the size) when the shape needs
 * more scratch than the array holds, before anything is enqueued.  All calls on one
 * device share its array and leave their contents in it (the kernels clear what must
 * start at zero), so calls that overlap on one device race: serialise them. */
verkv_status verkv_step_noalloc(const verkv_shape *s, const verkv_state *st, const float *q,
                                double beta, double eps, double delta, const void *K_host,
                                const void *V_host, verkv_step_out *out, int32_t *status,
                                verkv_stream_t stream);
size_t verkv_noalloc_scratch_bytes(void);

/* The memcpy form of the host fetch of KVFetch step 5 (picx.dev summary page,
 * "KVFETCH" step 5: the rows of F \ S move from CPU memory to the GPU; the abstract
 * page notes that these transfers can dominate decode latency).  The decode path does
 * not use it: verkv_refine reads those rows in place with zero-copy loads from its
 * kernels, which needs no host copy of the fetch list and no call per run.  This entry
 * point is the alternative for comparison, and for callers that want the rows
 * themselves: rows idx[0..count) of the row array `src` (row_bytes each) are copied
 * to dst[0..count) with one hipMemcpyAsync per run of consecutive indices, on
 * `stream`.
 *   src    pinned host memory (or device memory), not owned
 *   idx    [count] strictly ascending row indices >= 0, HOST memory (read during the
 *          call; a list produced by verkv_decode_step must be copied to the host first)
 *   dst    [count][row_bytes] device memory, written asynchronously
 *   runs   [host, may be NULL] number of copies issued
 * VERKV_EINVAL for NULL pointers, count < 0, row_bytes = 0 or a list that is not
 * strictly ascending (checked before any copy is issued); VERKV_EHIP if a copy cannot
 * be enqueued (copies issued before it stay enqueued). */
verkv_status verkv_gather_rows_memcpy(const void *src, size_t row_bytes, const int32_t *idx,
                                      int32_t count, void *dst, int64_t *runs,
                                      verkv_stream_t stream);

/* Optional kernel timing (instrumentation).  verkv_profile_begin creates 2*max_launches
 * HIP events (the only allocation the library makes, done here and not per step) and
 * turns recording on: every kernel launched afterwards by this library, up to
 * max_launches, is timed by an event pair that the dispatch itself stamps.  verkv_profile_report
 * waits for the recorded launches, writes per kernel kind the summed duration in ms
 * and the launch count (kinds: 0 PoissonComp, 1 pivot gather, 2 sketch scores,
 * 3 decision, 4 union/lists, 5 resident-pivot attention, 6 host-row attention,
 * 7 finish, 8 eps_after partials, 9 pivot coefficients, 10 staging copies, 11 2-bit
 * sketch quantiser, 12 re-solved cut, 13 staging plan), and
 * clears the record.  verkv_profile_end destroys the events.  Not
 * thread safe; meant for benchmarks. */
#define VERKV_PROFILE_KINDS 14
int32_t verkv_profile_begin(int32_t max_launches);
int32_t verkv_profile_report(double *total_ms, int32_t *launches, int32_t n_kinds);
void verkv_profile_end(void);

/* Waits for `stream` and reports problems the kernels of the last steps flagged in
 * `workspace` (a decode workspace): VERKV_OK, or VERKV_EHIP with verkv_last_error()
 * naming the condition (a team barrier that timed out, a fixed-point iteration that
 * did not converge).  Clears the flags. */
verkv_status verkv_check(void *workspace, const verkv_shape *s, int32_t cap, verkv_stream_t stream);

/* Human-readable name of a status code (static storage). */
const char *verkv_status_str(int32_t status);
/* Last HIP error text recorded on this thread ("" if none; static thread storage). */
const char *verkv_last_error(void);
/* ABI version: 100 * major + minor. */
int32_t verkv_version(void);
/* Identity of this build (static storage): the hex SHA-256 that the build script takes
 * over the library's sources, this header and the compiler flags, so a loaded library
 * can be checked against the sources it was built from ("unknown" if built without). */
const char *verkv_source_hash(void);

#ifdef __cplusplus
}
#endif
#endif /* VERKV_H */
