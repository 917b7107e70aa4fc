/*
 * specverify.h -- C ABI of the speculative-decoding verify step for AMD
 * Instinct MI355X (gfx950).
 *
 * Two calls make one verify step:
 *
 *   spec_verify_attn    grouped-query attention of the K+1 verifier query
 *                       positions (the last accepted token x0 and the drafts
 *                       d_1..d_K) over a paged KV cache, causal inside the
 *                       draft window.  The verifier checks every draft in
 *                       one forward pass over prefix + drafts (AI
 *                       Engineering from Scratch, "Speculative decoding and
 *                       EAGLE-3", section "Concept"; devpost "phoenix",
 *                       "What it does").
 *
 *   spec_reject_sample  the lossless rejection-sampling verifier over the
 *                       full vocabulary, then the commit of each sequence's
 *                       logical KV length (same lesson: "Concept", "Rolling
 *                       back the KV cache", "Build it" steps 1-4;
 *                       quickscale.ai "Quand et pourquoi utiliser le
 *                       speculative decoding", section 2).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument of the compute calls is device memory owned by
 *    the caller.  The library allocates no device memory, frees nothing and
 *    keeps no mutable global state; scratch memory is the caller's
 *    workspace.  The one exception is spec_reject_sample_noalloc, whose
 *    workspace is a fixed device array of the library (one per device).
 *    The host page pool (spec_pages_*) is host state owned by its handle.
 *  - Calls are asynchronous on `hip_stream` (a hipStream_t; NULL = the
 *    default stream).  Argument errors are detected on the host and
 *    returned before anything is launched.  A failed launch returns
 *    SV_ERR_HIP.  Device faults surface at the caller's next
 *    synchronisation.
 *  - Return value: SV_OK (0) or a negative sv_status.
 *  - dtype: SV_F32 or SV_BF16 (bf16 carried as 16-bit patterns).  All
 *    floating tensors of one call share the dtype.
 *  - Out-of-range indices in the inputs (block ids, draft tokens) never
 *    make the kernels read outside the buffers described here: they are
 *    clamped, and the results for such inputs are unspecified.
 *  - Validation mode: with SPECVERIFY_VALIDATE=1 in the environment (read
 *    at every call) each compute call first waits for its stream, copies
 *    its index, length, uniform, temperature and logit inputs to host
 *    memory and checks the preconditions stated for it (page ids of every
 *    page it touches in [0, num_blocks), lengths within capacity, tokens in
 *    [0, V), uniforms in [0, 1), finite temperatures and top-p values,
 *    logits without NaN or +inf and with a finite entry per row).  The
 *    first violation is printed to stderr and returned as SV_ERR_BAD_INPUT
 *    before anything is launched; after its launches the call waits for the
 *    stream again, so a device error is returned (SV_ERR_HIP) by the call
 *    that caused it.  A debugging aid: synchronous and slow.
 */
#ifndef SPECVERIFY_H_
#define SPECVERIFY_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SV_OK = 0,
  SV_ERR_INVALID_ARG = -1, /* null pointer, negative size, bad enum       */
  SV_ERR_UNSUPPORTED = -2, /* a shape outside the supported set          */
  SV_ERR_WORKSPACE = -3,   /* workspace smaller than the *_workspace_bytes */
  SV_ERR_HIP = -4,         /* a HIP runtime call or launch failed         */
  SV_ERR_NO_PAGES = -5,    /* the page pool has too few free pages        */
  SV_ERR_BAD_INPUT = -6    /* SPECVERIFY_VALIDATE=1: a device input breaks a
                              precondition (message on stderr)            */
} sv_status;

typedef enum { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

#define SV_BLOCK_SIZE 16 /* tokens per KV page */
#define SV_MAX_K 16      /* largest draft length accepted */

/* Window source of spec_verify_attn_window. */
#define SV_WINDOW_READ 0   /* read the window K/V from k_new / v_new only */
#define SV_WINDOW_APPEND 1 /* ... and store them into their cache slots */

/*
 * spec_verify_attn -- window-causal GQA of the K+1 verify positions.
 *
 * For sequence b with committed length L0 = kv_len[b], query position
 * i in [0, K] sits at absolute position t = L0 + i and attends keys
 * j in [0, t].  Query head h reads KV head g = h / (Hq / Hkv).
 * out = softmax(scale * q k^T) v, softmax in fp32.  The caller has already
 * written the window's own K/V (positions L0..L0+K) into the cache.
 *
 * Layouts (row-major, contiguous):
 *   q, out       [B, K+1, Hq, D]
 *   k_cache      [num_blocks, Hkv, D/X, 16, X]   X = 16 bytes / element
 *                (8 for bf16, 4 for fp32): 16-byte chunks of one key's
 *                head vector, the 16 tokens of a page side by side
 *   v_cache      [num_blocks, Hkv, D, 16]        one value coordinate of
 *                the 16 tokens of a page side by side
 *   block_table  [B, max_blocks_per_seq] int32: token j of sequence b is
 *                slot j % 16 of page block_table[b][j / 16]
 *   kv_len       [B] int32, L0 per sequence (read only here)
 *
 * Sizes: 1 <= K <= SV_MAX_K; D in {64, 128}; block_size == 16;
 *   Hq % Hkv == 0 and (Hq / Hkv) * (K + 1) <= 64; B >= 0 (B == 0 is a
 *   no-op); kv_len[b] + K + 1 <= min(max_kv_len + K + 1,
 *   16 * max_blocks_per_seq) for every b.
 * scale <= 0 selects 1 / sqrt(D).
 * workspace: at least spec_verify_attn_workspace_bytes(...) bytes of device
 *   memory (any content; 256-byte aligned), or NULL when that size is 0.
 */
int spec_verify_attn(const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_table, const int32_t* kv_len,
                     void* out, int B, int K, int Hq, int Hkv, int D,
                     int block_size, int num_blocks, int max_blocks_per_seq,
                     int max_kv_len, float scale, int dtype, void* workspace,
                     size_t workspace_bytes, void* hip_stream);

size_t spec_verify_attn_workspace_bytes(int B, int K, int Hq, int Hkv, int D,
                                        int max_kv_len);

/*
 * spec_verify_attn_tree -- the same attention over a flattened draft tree
 * (thakicloud, "speedup went from 1.4x to 0.8x", "Grading every branch in one
 * pass"; AI Engineering from Scratch, "Speculative decoding and EAGLE-3",
 * tree attention with a mask that follows the tree).
 *
 * The window holds N = K + 1 tree nodes; node 0 is the root (the last
 * accepted token) and node i's K/V sit at absolute position L0 + i.  Node i
 * attends keys [0, L0) and the window keys L0 + j for every j whose bit is
 * set in anc[b][i]: its ancestors and itself.  A chain (anc[b][i] =
 * 2^(i+1) - 1) is exactly spec_verify_attn.
 *
 * anc: [B, N] uint32 device array (bits above N - 1 ignored).  Every other
 *   argument, layout, size limit and error is as for spec_verify_attn with
 *   K = N - 1; the workspace is spec_verify_attn_workspace_bytes(B, N - 1,
 *   Hq, Hkv, D, max_kv_len).  anc == NULL with B > 0, or N < 2, is
 *   SV_ERR_INVALID_ARG.
 */
int spec_verify_attn_tree(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, const int32_t* kv_len,
                          const uint32_t* anc, void* out, int B, int N, int Hq,
                          int Hkv, int D, int block_size, int num_blocks,
                          int max_blocks_per_seq, int max_kv_len, float scale,
                          int dtype, void* workspace, size_t workspace_bytes,
                          void* hip_stream);

/*
 * spec_verify_attn_window -- the same attention, with the window's K/V taken
 * from the projection output instead of the cache (AI Engineering from
 * Scratch, "Speculative decoding and EAGLE-3", "Rolling back the KV cache":
 * verification extends the cache by the window, either written into a
 * scratch buffer and committed on acceptance, or written in place and rolled
 * back by the logical length; sglang_spec_decode README, the provisional KV
 * layer).
 *
 * k_new, v_new: [B, N, Hkv, D] (dtype), row i = window position L0 + i (chain)
 *   or tree node i; device memory, 16-byte aligned, read only.
 * mode SV_WINDOW_READ: the window keys are read from k_new / v_new and the
 *   cache is not written (the scratch-buffer variant: spec_kv_commit moves
 *   the accepted rows into the cache afterwards).
 * mode SV_WINDOW_APPEND: row i is stored into its cache slot L0 + i (pages
 *   from block_table; the caller has reserved them) by a copy kernel the call
 *   launches first, and the attention then reads the whole window from the
 *   cache, exactly as spec_verify_attn (the same output bit for bit).  The
 *   copy moves 16-byte vectors: k_new, v_new and both caches 16-byte aligned
 *   (either dtype), else SV_ERR_INVALID_ARG.
 * anc: NULL for a chain (N = K + 1), or [B, N] ancestor sets of a tree as for
 *   spec_verify_attn_tree.  Everything else as spec_verify_attn with
 *   K = N - 1 (same workspace).  out and the cache slots L0 .. L0 + N - 1 are
 *   the only memory written.  N < 2, a bad mode, or NULL k_new / v_new with
 *   B > 0 is SV_ERR_INVALID_ARG.
 */
int spec_verify_attn_window(const void* q, const void* k_new, const void* v_new,
                            void* k_cache, void* v_cache, const int32_t* block_table,
                            const int32_t* kv_len, const uint32_t* anc, void* out,
                            int B, int N, int Hq, int Hkv, int D, int block_size,
                            int num_blocks, int max_blocks_per_seq, int max_kv_len,
                            float scale, int dtype, int mode, void* workspace,
                            size_t workspace_bytes, void* hip_stream);

/*
 * spec_reject_sample -- lossless verifier over the full vocabulary plus the
 * KV-length commit.
 *
 * Rows: target row i (i = 0..K) is q_{i+1}, the verifier's distribution
 * after x0, d_1..d_i; draft row i (i = 0..K-1) is p_{i+1}, the law d_{i+1}
 * was drawn from.  Both share one vocabulary of size V.
 *
 * Sampling (temperature[b] > 0): q = softmax(target / T), p =
 * softmax(draft / T).  d_i is accepted iff p_i(d_i) == 0 or
 * u[i-1] < min(1, q_i(d_i) / p_i(d_i)); n = the number of leading accepts.
 * If n < K the emitted token is drawn from (q_{n+1} - p_{n+1})_+ (from
 * q_{n+1} if that has zero mass); if n == K from q_{K+1} (bonus).  The draw
 * is the smallest v with C(v) > u[K] * Z, C the inclusive prefix sum of the
 * weights and Z their total (the largest positive-weight v if rounding
 * leaves none).
 * Greedy (temperature[b] <= 0, or draft_logits == NULL): d_i is accepted iff
 * it equals argmax(target row i-1) (lowest index on ties); the emitted
 * token is argmax(target row n).  Draft logits are not read.
 *
 * Outputs: out_tokens[b] = d_1..d_n, the emitted token, then -1;
 * num_accepted[b] = n; kv_len[b] += n + 1 (x0 plus the accepted drafts stay,
 * the K - n rejected slots are rolled back).  The call is therefore NOT
 * idempotent: retrying it needs kv_len restored first.
 * counters (optional, NULL to skip): counters[0] += K and
 * counters[1] += n for every sequence (proposed / accepted drafts).
 *
 * Layouts (row-major, contiguous):
 *   target_logits [B, K+1, V]; draft_logits [B, K, V] (dtype)
 *   draft_tokens  [B, K] int32 in [0, V)
 *   uniforms      [B, K+1] float32 in [0, 1)
 *   temperature   [B] float32
 *   out_tokens    [B, K+1] int32; num_accepted [B] int32; kv_len [B] int32
 * Preconditions: every row holds at least one finite logit and no NaN or
 * +inf; -inf logits are allowed (probability 0).
 * Sizes: 1 <= K <= SV_MAX_K; 1 <= V < 2^31 / 4; B >= 0 (B == 0 is a no-op);
 *   B * (2K+1) < 2^31.
 * workspace: at least spec_reject_sample_workspace_bytes(B, K, V) bytes of
 *   device memory (any content; 256-byte aligned).
 */
int spec_reject_sample(const void* target_logits, const void* draft_logits,
                       const int32_t* draft_tokens, const float* uniforms,
                       const float* temperature, int32_t* out_tokens,
                       int32_t* num_accepted, int32_t* kv_len,
                       unsigned long long* counters, int B, int K, int V,
                       int dtype, void* workspace, size_t workspace_bytes,
                       void* hip_stream);

size_t spec_reject_sample_workspace_bytes(int B, int K, int V);

/*
 * spec_reject_sample_noalloc -- spec_reject_sample for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the workspace is a file-scope device
 * array of the library instead of a caller buffer.  The call itself allocates
 * nothing and calls no allocating routine; the caller still provides every
 * input and output.
 *
 * Arguments, layouts, results and errors are those of spec_reject_sample
 * without workspace / workspace_bytes.  Limit: spec_reject_sample_workspace_
 * bytes(B, K, V) <= SV_NOALLOC_SCRATCH_BYTES (16 MiB: B = 256, K = 7,
 * V = 128256 needs 5.4 MB), else SV_ERR_WORKSPACE and nothing is launched.
 * Each device the library runs on holds its own copy of the array until the
 * process ends; its address is looked up on the first call made with that
 * device current (a failure there is SV_ERR_HIP).  The array keeps the last
 * call's contents and needs no clearing.  Every call on one device shares
 * that device's array: calls that overlap on one device (different streams,
 * or host threads, without ordering between them) race and give undefined
 * results; calls ordered on one stream are fine.  Validation mode
 * (SPECVERIFY_VALIDATE) does not apply to this call: it stages inputs in
 * host memory.
 */
#define SV_NOALLOC_SCRATCH_BYTES (16u << 20)
int spec_reject_sample_noalloc(const void* target_logits, const void* draft_logits,
                               const int32_t* draft_tokens, const float* uniforms,
                               const float* temperature, int32_t* out_tokens,
                               int32_t* num_accepted, int32_t* kv_len,
                               unsigned long long* counters, int B, int K, int V, int dtype,
                               void* hip_stream);

/*
 * spec_reject_sample_filtered -- spec_reject_sample with top-k / top-p
 * filtering of both laws before the verifier (quickscale.ai, "Quand et
 * pourquoi utiliser le speculative decoding", "Influence du sampling": top-p
 * and top-k shape the drafted tokens and the acceptance).
 *
 * Per sampling sequence b, with the logits divided by T: top-k keeps the
 * tokens whose logit is >= the k-th largest (ties kept; top_k[b] <= 0 or
 * >= V: off); then top-p keeps, among those, the tokens whose logit is >= v*,
 * v* the largest logit value whose set {x >= v*} holds at least top_p[b] of
 * the kept mass (ties kept; top_p[b] <= 0 or >= 1: off).  Every target row and
 * every draft row is filtered with the sequence's own parameters and
 * renormalised, and the verifier runs on the filtered laws q', p' (accept
 * with min(1, q'(d)/p'(d)), p'(d) = 0 accepts, residual (q' - p')_+, bonus
 * from q'): the emitted tokens follow the filtered target.  The drafts are
 * expected to come from the filtered draft law.  Greedy sequences are
 * unaffected (the argmax is always kept).
 *
 * top_k [B] int32, top_p [B] float32 device arrays; either may be NULL (off
 * for every sequence).  The top-p set is chosen on masses summed in 40-bit
 * fixed point from fp32 weights, so a boundary within ~1e-6 of top_p may be
 * decided differently from an exact computation.  Everything else is as
 * for spec_reject_sample.
 *
 * workspace: at least spec_reject_sample_workspace_bytes(B, K, V) bytes;
 *   with spec_reject_sample_filtered_workspace_bytes(B, K, V) bytes a bf16
 *   call whose rows start on 16-byte boundaries (V % 8 == 0) also counts, in
 *   its one sweep over the rows, every value of a window of bf16 keys placed
 *   from a fixed sample's maximum (512 keys with top-k, 1024 for top-p
 *   alone, reaching six binades under it), and each filtered row whose thresholds
 *   fall inside that window needs no pass of its own; other rows (and every
 *   row with the smaller workspace, or fp32 logits) take the filter's radix
 *   passes: one or two extra reads of the row per active filter (bf16; up
 *   to four for fp32).  The results are the same either way, except inside
 *   the top-p band above.
 */
int spec_reject_sample_filtered(const void* target_logits, const void* draft_logits,
                                const int32_t* draft_tokens, const float* uniforms,
                                const float* temperature, const int32_t* top_k,
                                const float* top_p, int32_t* out_tokens,
                                int32_t* num_accepted, int32_t* kv_len,
                                unsigned long long* counters, int B, int K, int V,
                                int dtype, void* workspace, size_t workspace_bytes,
                                void* hip_stream);

/* Workspace of spec_reject_sample_filtered with room for the sweep's window
 * (0 for invalid sizes). */
size_t spec_reject_sample_filtered_workspace_bytes(int B, int K, int V);

/*
 * spec_reject_sample_tree -- the lossless verifier over a flattened draft
 * tree, plus the KV commit (AI Engineering from Scratch, "Speculative
 * decoding and EAGLE-3": EAGLE-2's draft tree, the accept test and residual
 * of "Concept"; thakicloud, "Grading every branch in one pass": every branch
 * is graded in one forward pass and the surviving path is kept).
 *
 * The tree: N nodes, node 0 the root (the last accepted token), parent[i] < i
 * for i >= 1; its shape is shared by the whole batch.  Target row v is q_v,
 * the verifier's distribution after the path to node v; draft row v is p_v,
 * the law node v's children were drawn from (each independently).  Walking
 * from the root with q' = q_v:
 *   - the children c of v are tested in increasing index order: accept c iff
 *     p_v(d_c) <= 0 or u[c] < min(1, q'(d_c) / p_v(d_c));
 *   - after a rejected child, q' <- (q' - p_v)_+ normalised (recursive
 *     rejection sampling; a zero-mass residual leaves q' unchanged);
 *   - the first accepted child is emitted and becomes v (q' <- q_v);
 *   - when every child of v is rejected, or v is a leaf, the final token is
 *     drawn from q' by inverse CDF with u[0], as in spec_reject_sample.
 * The emitted token at every node then has exactly the law q_v.  A chain
 * (parent[i] = i - 1) gives exactly spec_reject_sample with u[i] <-> u_{i-1}
 * and u[0] <-> u_K.  Greedy (temperature[b] <= 0, or draft_logits == NULL):
 * the first child whose token equals argmax(q_v) (lowest index on ties) is
 * accepted, else argmax(q_v) is emitted and the walk ends.
 *
 * Outputs: out_tokens[b] = tokens of the accepted nodes along the path, the
 * final token, then -1; out_nodes[b] = the accepted node indices, then -1;
 * num_accepted[b] = n; kv_len[b] += n + 1.  The caller moves the K/V of the
 * accepted nodes (slots L0 + out_nodes[b][j]) to positions L0 + 1 + j.  Not
 * idempotent (kv_len).  counters (optional): counters[0] += N - 1 and
 * counters[1] += n per sequence.
 *
 * Layouts (row-major, contiguous):
 *   parent        [N] int32 HOST array (parent[0] = -1)
 *   target_logits [B, N, V]; draft_logits [B, N, V] (rows of leaves unread)
 *   tokens        [B, N] int32 (entry 0 unused), in [0, V)
 *   uniforms      [B, N] float32 in [0, 1): u[i] tests node i, u[0] the final draw
 *   temperature   [B] float32
 *   out_tokens, out_nodes [B, N] int32; num_accepted [B] int32; kv_len [B] int32
 * Preconditions as for spec_reject_sample.  Sizes: 1 <= N <= SV_MAX_K + 1;
 *   1 <= V < 2^31 / 4; B >= 0 (B == 0 is a no-op); B * (2N - 1) < 2^31.
 *   A parent array that is not a tree in topological order is
 *   SV_ERR_INVALID_ARG.
 * Work: one exact float64 pass over a node's row pair per rejection (and one
 *   for a leaf's bonus draw), in rounds; the number of rounds follows from
 *   the shape (the largest number of passes any walk can need).
 * workspace: at least spec_reject_sample_tree_workspace_bytes(B, N, V) bytes
 *   of device memory (any content; 256-byte aligned).
 */
int spec_reject_sample_tree(const void* target_logits, const void* draft_logits,
                            const int32_t* parent, const int32_t* tokens,
                            const float* uniforms, const float* temperature,
                            int32_t* out_tokens, int32_t* out_nodes,
                            int32_t* num_accepted, int32_t* kv_len,
                            unsigned long long* counters, int B, int N, int V,
                            int dtype, void* workspace, size_t workspace_bytes,
                            void* hip_stream);

size_t spec_reject_sample_tree_workspace_bytes(int B, int N, int V);

/*
 * spec_reject_sample_tree_filtered -- spec_reject_sample_tree with top-k /
 * top-p filtering of the laws before the walk (quickscale.ai, "Quand et
 * pourquoi utiliser le speculative decoding", "Influence du sampling", with
 * the tree verifier of thakicloud, "Grading every branch in one pass").
 *
 * The filters of spec_reject_sample_filtered, with the sequence's own
 * (top_k[b], top_p[b]), on every target row q_v and on the draft row p_v of
 * every node with children (leaf draft rows are never read); the walk then
 * runs unchanged on the filtered laws q', p': a child whose token is outside
 * p'_v's kept set passes (p'(d) = 0), one outside q'_v's set fails unless it
 * also is outside p'_v's, the sibling residuals are (q' - p')_+ and the final
 * draw is from the filtered law.  Greedy sequences are unaffected.
 *
 * top_k [B] int32, top_p [B] float32 device arrays; either may be NULL (off
 * for every sequence).  The same top-p boundary band as the chain call.
 * workspace: spec_reject_sample_tree_workspace_bytes(B, N, V), or
 *   spec_reject_sample_tree_filtered_workspace_bytes(B, N, V) for the
 *   sweep's window (as spec_reject_sample_filtered).  Everything else is as
 *   for spec_reject_sample_tree.
 */
int spec_reject_sample_tree_filtered(const void* target_logits, const void* draft_logits,
                                     const int32_t* parent, const int32_t* tokens,
                                     const float* uniforms, const float* temperature,
                                     const int32_t* top_k, const float* top_p,
                                     int32_t* out_tokens, int32_t* out_nodes,
                                     int32_t* num_accepted, int32_t* kv_len,
                                     unsigned long long* counters, int B, int N, int V,
                                     int dtype, void* workspace, size_t workspace_bytes,
                                     void* hip_stream);

/* Workspace of spec_reject_sample_tree_filtered and spec_reject_sample_trees
 * with room for the sweep's window (0 for invalid sizes). */
size_t spec_reject_sample_tree_filtered_workspace_bytes(int B, int N, int V);

/*
 * spec_reject_sample_trees -- spec_reject_sample_tree_filtered with one tree
 * per sequence (thakicloud, "Grading every branch in one pass": each request
 * grades its own draft tree; AI Engineering from Scratch, "Speculative
 * decoding and EAGLE-3": EAGLE-2 grows a tree per context).  Sequence b's
 * tree is parents[b]; everything the shared-tree calls define (the walk, the
 * outputs, the commit, the filters and their band) applies per sequence with
 * that tree.  All trees have N nodes (the shape of spec_verify_attn_tree's
 * ancestor sets).
 *
 * parents: [B, N] int32 DEVICE array, parents[b][0] = -1 and
 *   0 <= parents[b][i] < i; a parent outside [0, i) is read as i - 1 (with
 *   SPECVERIFY_VALIDATE=1 it is SV_ERR_BAD_INPUT).  NULL only with B == 0.
 * top_k, top_p: as spec_reject_sample_tree_filtered, or NULL (no filter).
 * Work: the sweep and filters skip the draft rows of a sequence's leaves; the
 *   host cannot see the shapes, so it launches N - 1 rounds (the most a tree
 *   of N nodes can need: a root with N - 1 children), and a sequence whose
 *   walk has ended leaves the remaining rounds at once.
 * workspace: spec_reject_sample_tree_workspace_bytes(B, N, V) (it includes
 *   room for the B shapes), or spec_reject_sample_tree_filtered_workspace_
 *   bytes(B, N, V) for the sweep's window with filters.  Other sizes and
 *   errors as spec_reject_sample_tree.
 */
int spec_reject_sample_trees(const void* target_logits, const void* draft_logits,
                             const int32_t* parents, const int32_t* tokens, const float* uniforms,
                             const float* temperature, const int32_t* top_k, const float* top_p,
                             int32_t* out_tokens, int32_t* out_nodes, int32_t* num_accepted,
                             int32_t* kv_len, unsigned long long* counters, int B, int N, int V,
                             int dtype, void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * spec_kv_commit -- after the verifier, the surviving window rows' K/V into
 * their committed positions (AI Engineering from Scratch, "Speculative
 * decoding and EAGLE-3", "Rolling back the KV cache": a scratch buffer
 * committed on acceptance, or the cache written in place; thakicloud,
 * "Grading every branch in one pass": the surviving tree path is kept).
 *
 * For sequence b, n = num_accepted[b] and L0 = kv_len[b] - n - 1 (kv_len as
 * the verifier left it).  Surviving row j = 0..n is the root (j = 0), then
 * the accepted nodes in path order: nodes[b][j - 1] for a tree (out_nodes of
 * spec_reject_sample_tree), row j for a chain (nodes == NULL).  Row j goes
 * to position L0 + j, read from k_src / v_src [B, N, Hkv, D] (scratch mode)
 * or, with k_src == v_src == NULL, from its window slot L0 + row of the
 * cache (in place: a tree's path is compacted; every source is read before
 * any slot is written; a chain in place has nothing to move and launches
 * nothing).  The emitted token's K/V are not committed here: the next
 * verify call writes them as its root.  Sequences with num_accepted outside
 * [0, N) are skipped.
 *
 * Layouts as spec_verify_attn; nodes [B, N] int32.  Sizes: 1 <= N <=
 * SV_MAX_K + 1, D in {64, 128}, block_size == 16.  Only the cache slots
 * L0 .. L0 + n are written.  Keys, runs of values and scratch rows move as
 * 16-byte vectors: both caches and k_src / v_src 16-byte aligned, else
 * SV_ERR_INVALID_ARG.
 */
int spec_kv_commit(void* k_cache, void* v_cache, const int32_t* block_table,
                   const int32_t* kv_len, const int32_t* num_accepted,
                   const int32_t* nodes, const void* k_src, const void* v_src,
                   int B, int N, int Hkv, int D, int block_size, int num_blocks,
                   int max_blocks_per_seq, int dtype, void* hip_stream);

/*
 * spec_pages_* -- host-side KV page list with provisional window pages (AI
 * Engineering from Scratch, "Rolling back the KV cache"; sglang_spec_decode
 * README, the provisional KV layer).  Host memory only, no GPU calls.
 *
 * A sequence owns pages for positions [0, 16 * pages).  reserve(seq, len)
 * grows that to cover positions [0, len) (call it with L0 + N before a
 * verify; the new pages are provisional), taking the lowest-numbered free
 * pages first; commit(seq, len) frees every page whose first position is at
 * or past len (the pages only a rejected tail used, or an explicit rollback)
 * and keeps the rest; release(seq) frees them all.  block_table() is the
 * [max_seqs, max_blocks_per_seq] int32 host table the verify calls need
 * (unused entries 0), valid until the next call on the pool.  check()
 * verifies that every page is owned exactly once (by one sequence or the
 * free list).  Errors: SV_ERR_INVALID_ARG (bad sequence or length, a length
 * past max_blocks_per_seq pages, a commit past the reserved pages),
 * SV_ERR_NO_PAGES (reserve needs more free pages than there are; nothing is
 * taken).  Not thread-safe.
 */
typedef struct sv_page_pool sv_page_pool;
sv_page_pool* spec_pages_create(int num_blocks, int max_seqs, int max_blocks_per_seq);
void spec_pages_destroy(sv_page_pool* pool);
int spec_pages_reserve(sv_page_pool* pool, int seq, int total_len);
int spec_pages_commit(sv_page_pool* pool, int seq, int committed_len);
int spec_pages_release(sv_page_pool* pool, int seq);
int spec_pages_free_count(const sv_page_pool* pool);
int spec_pages_seq_blocks(const sv_page_pool* pool, int seq);
const int32_t* spec_pages_block_table(const sv_page_pool* pool);
int spec_pages_check(const sv_page_pool* pool);

/*
 * spec_bandit_* -- host-side draft-length controller (devpost "phoenix",
 * "How we built it", "The bandit").  Arms are indices 0..n_arms-1 into the
 * caller's list of draft lengths (the page uses {0, 2, 4, 6, 8}).  The first
 * warmup_rounds * n_arms decisions visit the arms in order; after that,
 * decision t explores with probability max(0.05, 0.3 * 0.97^t) (t counts
 * every earlier decision), picking arm floor(u_arm * n_arms), and otherwise
 * takes the arm with the highest running-average reward (lowest index on
 * ties).  u_explore and u_arm in [0, 1) are the caller's random numbers.
 * update() adds one reward (the caller's measured output tokens per second)
 * to the running mean of its arm and advances t.  select() returns the arm
 * index or SV_ERR_INVALID_ARG.  Host memory only; not thread-safe.
 *
 * spec_accept_stats -- from a verify call's num_accepted (HOST copy, [B]):
 * a[i-1] = fraction of sequences with n >= i for i = 1..K (per-position
 * acceptance, quickscale.ai section 4) and mean_len = mean(n + 1), the
 * tokens emitted per verify.
 */
typedef struct sv_bandit sv_bandit;
sv_bandit* spec_bandit_create(int n_arms, int warmup_rounds);
void spec_bandit_destroy(sv_bandit* bandit);
int spec_bandit_select(const sv_bandit* bandit, double u_explore, double u_arm);
int spec_bandit_update(sv_bandit* bandit, int arm, double reward);
int spec_bandit_stats(const sv_bandit* bandit, long long* pulls, double* means,
                      long long* t);
int spec_accept_stats(const int32_t* num_accepted, int B, int K, double* a,
                      double* mean_len);

/*
 * spec_read_probe -- a measurement aid, not part of the verify path: reads
 * `bytes` of device memory at `buf` once with the sweep's access pattern
 * (16-byte nontemporal loads, 1 KB contiguous per wave instruction, eight in
 * flight per lane) over `grid` workgroups of 256 threads, and writes one
 * checksum word per workgroup to `sink` [grid] (device memory).  Timing it
 * gives the streaming-read bandwidth this chip reaches, against which the
 * verify kernels' rates are also reported.  bytes must be a positive
 * multiple of 8192 and buf 16-byte aligned; 1 <= grid <= 2^20; otherwise
 * SV_ERR_INVALID_ARG.  Asynchronous on hip_stream.
 */
int spec_read_probe(const void* buf, size_t bytes, uint32_t* sink, int grid, void* hip_stream);

/* Static description of a status code. */
const char* spec_status_string(int status);

/* Library version as major * 10000 + minor * 100 + patch. */
int spec_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H_ */
