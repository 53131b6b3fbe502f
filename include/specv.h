/*
 * specv -- the verify step of speculative decoding on AMD MI355X (gfx950).
 *
 * The verify step as three operations, each asynchronous on the caller's HIP
 * stream:
 *
 *   specv_build_tree_mask   ancestor mask and depth of every draft node, from
 *                           a parent array;
 *   specv_tree_attn_verify  the target's attention for all draft nodes in one
 *                           pass over the KV cache, each node seeing the
 *                           committed context plus its own ancestors;
 *   specv_accept_resample   the exact accept / reject / resample rule over the
 *                           vocabulary, for chains and for trees, greedy at
 *                           temperature 0;
 * and the steps around them:
 *   specv_tree_expand       one level of draft-tree construction (top-k
 *                           children kept by cumulative draft probability);
 *   specv_kv_commit         keep the accepted path's KV-cache rows, drop the
 *                           rejected branches';
 *   specv_verify_layer      one whole target-model layer over the draft nodes
 *                           (projections, rotary encoding at the tree
 *                           positions, the tree attention above, gated MLP);
 *   specv_pack_weights, specv_verify_layer_packed   the same layer on weights
 *                           stored in the tile order its products read.
 *
 * Sources (web pages on speculative decoding):
 *   [SD-review] paper review of Leviathan, Kalman, Matias, "Fast Inference
 *               from Transformers via Speculative Decoding" (ICML 2023);
 *   [PTD]       technical summary of "Progressive Tree Drafting (PTD)";
 *   [SD-EAGLE]  lesson "Speculative Decoding and EAGLE".
 *
 * Conventions shared by all calls
 *   - K is the number of draft nodes; every per-node array has K + 1 rows,
 *     row 0 being the root (the last committed token), rows 1..K the drafts.
 *     A chain of K drafts is the parent array {-1, 0, 1, ..., K-1}.
 *   - Parent arrays are topological: parent[0] = -1 and 0 <= parent[i] < i.
 *   - All pointers are DEVICE pointers unless stated otherwise, contiguous,
 *     row-major, 16-byte aligned for the logits / q / k / v / out buffers.
 *   - The caller owns every buffer, including the workspace (size from the
 *     *_workspace_bytes queries).  The library allocates nothing, frees
 *     nothing and never synchronises the stream; it keeps no state between
 *     calls except the text of the last error of the calling thread.
 *   - Argument errors are detected on the host and returned before any
 *     launch; nothing is written then.  Errors that depend on device data
 *     (a bad parent array, an out-of-range token or context length) are
 *     reported per sequence in the outputs, as described per call.
 *   - B == 0 is a valid empty call: SPECV_OK, no launch.
 *   - Outputs are a pure function of the inputs (and of seed and offset for
 *     the accept rule): calls replay bit-exactly.
 */
#ifndef SPECV_H
#define SPECV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SPECV_OK = 0,
    SPECV_ERR_INVALID_ARG = 1,   /* NULL pointer, size out of range, bad temperature, ... */
    SPECV_ERR_UNSUPPORTED = 2,   /* a head size, dtype or size the kernels do not cover */
    SPECV_ERR_WORKSPACE = 3,     /* workspace NULL or smaller than the query returns */
    SPECV_ERR_HIP = 4,           /* a kernel launch failed; see specv_last_error() */
    /* not statuses: they make every 32-bit value a valid value of the type, so that a value
       outside the list (passed in from C, say) is an ordinary unknown value in C++ too */
    SPECV_STATUS_RANGE_LOW_ = -0x7fffffff - 1,
    SPECV_STATUS_RANGE_HIGH_ = 0x7fffffff
} specv_status;

typedef enum {
    SPECV_F32 = 0,
    SPECV_BF16 = 1,
    /* not dtypes: every 32-bit value is a value of the type (an unknown one is rejected) */
    SPECV_DTYPE_RANGE_LOW_ = -0x7fffffff - 1,
    SPECV_DTYPE_RANGE_HIGH_ = 0x7fffffff
} specv_dtype;

/* Largest supported K + 1 and vocabulary size. */
#define SPECV_MAX_NODES 1024
#define SPECV_MAX_VOCAB (1 << 21)

/*
 * Ancestor mask of a draft tree.
 *
 * [SD-EAGLE] "Tree Attention Verification": the verify pass uses a causal
 * mask that encodes the tree, each node attending only to its ancestors;
 * [PTD] Method 1, "Attention Masking".  Bit j of row i is set iff j == i or
 * j is an ancestor of i (the causal diagonal is kept, so a chain gives the
 * lower-triangular mask).
 *
 *   parent       [B][K+1] int32
 *   mask         [B][K+1][W] uint32, W = (K + 32) / 32 words per row; bit
 *                (j % 32) of word j / 32 of row i  <=>  j in ancestors(i) u {i}
 *   depth        [B][K+1] int32, number of ancestors (root 0); position of a
 *                node in the sequence is ctx_len + depth
 *   tree_status  [B] int32: 0 if the parent array is valid, else the index of
 *                the first invalid entry + 1; an invalid sequence gets an
 *                all-zero mask and depth -1 everywhere.
 *
 * Errors: SPECV_ERR_INVALID_ARG for a NULL pointer, B < 0, K < 0 or
 * K + 1 > SPECV_MAX_NODES.
 */
specv_status specv_build_tree_mask(const int32_t* parent, int32_t B, int32_t K,
                                   uint32_t* mask, int32_t* depth, int32_t* tree_status,
                                   hipStream_t stream);

/*
 * Tree-attention verify: one layer's attention for all K + 1 node rows.
 *
 * [SD-EAGLE] "Tree Attention Verification": all nodes are verified in one
 * forward pass with the tree mask; [PTD] Method 4, "Verification";
 * [SD-review] §2 step 2: the target sees the context and all drafts at once.
 * For sequence b, node i, query head h (KV head h / (Hq / Hkv)):
 *   keys  = the context entries 0 .. ctx_len[b]-1 (all visible) and the tree
 *           entries ctx_len[b] + j for every j with mask bit (i, j) set;
 *   out   = softmax(scale * q . k) . v over those keys;
 *   lse   = natural log of the softmax denominator (sum of exp of the scaled
 *           scores), optional.
 *
 *   q        [B][K+1][Hq][D]       dtype
 *   k_cache  [B][Hkv][Lmax][D]     dtype; node j's own K/V row is at ctx_len[b] + j
 *   v_cache  [B][Hkv][Lmax][D]     dtype
 *   ctx_len  [B] int32             committed context length of each sequence
 *   mask     [B][K+1][W] uint32    from specv_build_tree_mask
 *   scale    score scale (pass 1/sqrt(D) for the usual attention)
 *   dtype    SPECV_BF16 (bf16 in, fp32 accumulation, bf16 out) or SPECV_F32
 *   out      [B][K+1][Hq][D]       dtype
 *   lse      [B][K+1][Hq] float32, or NULL
 *   workspace / workspace_bytes: at least specv_attn_workspace_bytes(...)
 *
 * A sequence with ctx_len[b] < 0 or ctx_len[b] + K + 1 > Lmax gets NaN in
 * out and lse (nothing outside the cache is read).
 * Errors: SPECV_ERR_INVALID_ARG (NULL pointer, sizes <= 0, Hq % Hkv != 0,
 * K + 1 > SPECV_MAX_NODES, Lmax < K + 1, non-finite scale),
 * SPECV_ERR_UNSUPPORTED (D not 64 or 128, unknown dtype),
 * SPECV_ERR_WORKSPACE, SPECV_ERR_HIP.
 */
specv_status specv_tree_attn_verify(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* ctx_len, const uint32_t* mask,
                                    int32_t B, int32_t K, int32_t Hq, int32_t Hkv, int32_t D,
                                    int32_t Lmax, float scale, specv_dtype dtype,
                                    void* out, float* lse,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);

size_t specv_attn_workspace_bytes(int32_t B, int32_t K, int32_t Hq, int32_t Hkv, int32_t D,
                                  int32_t Lmax);

/*
 * Exact accept / reject / resample over the vocabulary.
 *
 * [SD-EAGLE] "The Exactness Rule" and [SD-review] §2: p = softmax(target / T),
 * q = softmax(draft / T); a draft x is accepted if u < p(x) / q(x); at the
 * first rejection a replacement is drawn from (p - q)+ / ||(p - q)+||_1 and the
 * step stops; if every draft on the path is accepted a bonus token is drawn
 * from p of the last node.  T == 0 is the greedy rule: accept iff the draft
 * equals argmax p (lowest token id on ties), otherwise emit argmax p.
 * Trees ([PTD] Method 4, "Acceptance Logic"): at node v the children are
 * tested in increasing node index as draws without replacement from q_v; after
 * a rejection the target becomes the residual and the draft loses the
 * rejected token (renormalised).  Equivalently, after i rejections the target
 * is (p - c_i q)+ / R_i with c_0 = 0, R_0 = Q_0 = 1, c_{i+1} = c_i + R_i / Q_i,
 * Q the draft mass not yet rejected.  A child repeating an earlier sibling's
 * token is skipped.
 *
 *   target_logits [B][K+1][V]  row v is the target's next-token logits after node v
 *   draft_logits  [B][K+1][V]  row v is the draft distribution that proposed v's
 *                              children (rows of leaves are not read); may be NULL
 *                              iff temperature == 0
 *   logits_dtype  SPECV_F32 or SPECV_BF16 (both logits tensors)
 *   tokens        [B][K+1] int32; tokens[b][0] is the root token (not read)
 *   parent        [B][K+1] int32
 *   temperature   T >= 0, finite
 *   seed, offset  uniforms: Philox4x64-10 (Salmon et al., SC'11) with key
 *                 (seed, 0) and counter (node, b, offset, 0); word 0 is the
 *                 acceptance uniform of that node, word 1 the resampling
 *                 uniform if the walk ends there; a word w maps to
 *                 (2 * (w >> 12) + 1) * 2^-53.  Advance offset once per call.
 *   accept_len    [B] int32: number of accepted draft nodes; -1 if the parent
 *                 array is invalid or a draft token is outside [0, V).  The
 *                 result does not depend on how the device schedules the
 *                 call: the workgroups that share a sequence never wait on one
 *                 another for longer than a budget (100 us; environment
 *                 variable SPECV_ACCEPT_WAIT_US, read at each call, sets it
 *                 in microseconds), after which a workgroup computes the
 *                 values it waits for itself, bit for bit what their owner
 *                 computes.
 *   out_nodes     [B][K+1] int32: accepted node ids from the first level down,
 *                 then -1
 *   out_tokens    [B][K+1] int32: the accepted tokens, then the resampled /
 *                 bonus / greedy token (accept_len + 1 valid entries), then -1
 *   p_tok, q_tok  [B][K+1] float32 or NULL: p_parent(v)(tokens[v]) and
 *                 q_parent(v)(tokens[v]) for every v >= 1; NaN at v == 0, at
 *                 T == 0 and for invalid sequences
 *   workspace / workspace_bytes: at least specv_accept_workspace_bytes(...),
 *                 zero-filled by the caller before its first use; the calls
 *                 keep it valid afterwards (its first 128 bytes carry a launch
 *                 counter from call to call, so it is not cleared again, and a
 *                 call captured in a graph stays correct on every replay).
 *
 * Ownership: every pointer is device memory owned by the caller; the call only
 * enqueues work on `stream` and returns.  Calls that share a workspace must be
 * ordered on one stream.
 *
 * Errors: SPECV_ERR_INVALID_ARG (NULL pointer, B < 0, K < 0,
 * K + 1 > SPECV_MAX_NODES, V < 1 or V > SPECV_MAX_VOCAB, T < 0 or not finite,
 * draft NULL with T > 0), SPECV_ERR_UNSUPPORTED (dtype), SPECV_ERR_WORKSPACE,
 * SPECV_ERR_HIP.
 */
specv_status specv_accept_resample(const void* target_logits, const void* draft_logits,
                                   specv_dtype logits_dtype,
                                   const int32_t* tokens, const int32_t* parent,
                                   int32_t B, int32_t K, int32_t V, float temperature,
                                   uint64_t seed, uint64_t offset,
                                   int32_t* accept_len, int32_t* out_tokens, int32_t* out_nodes,
                                   float* p_tok, float* q_tok,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

size_t specv_accept_workspace_bytes(int32_t B, int32_t K, int32_t V, specv_dtype logits_dtype);

/*
 * How the siblings of a tree node were drafted.  The accept rule stays the
 * recursive rejection rule; what changes is the proposal each sibling is
 * taken to be drawn from, and the rule is exact only for the drafting it
 * names.  [PTD] Method 4, "Acceptance Logic" (sampling without replacement);
 * [SD-EAGLE] "EAGLE: tree drafting and feature reuse" (K candidates per depth).
 */
typedef enum {
    /* drawn without replacement from q_v (the rule of specv_accept_resample):
       after a rejection the draft loses the rejected token, renormalised; a
       repeated token is skipped */
    SPECV_SIBLINGS_WITHOUT_REPLACEMENT = 0,
    /* drawn independently from q_v: the proposal stays q_v, so after i
       rejections the target is (p - c_i q)+ / R_i with c_{i+1} = c_i + R_i;
       repeated tokens are tested (and rejected) like any other */
    SPECV_SIBLINGS_IID = 1,
    /* fixed candidates (e.g. the draft's top-k), each a point mass: accept x
       with probability p'(x); after a rejection p' is p without the rejected
       tokens, renormalised, and the final draw is from it; the draft logits
       are not read (may be NULL) and q_tok is NaN */
    SPECV_SIBLINGS_DETERMINISTIC = 2,
    /* not rules: every 32-bit value is a value of the type (an unknown one is rejected) */
    SPECV_SIBLINGS_RANGE_LOW_ = -0x7fffffff - 1,
    SPECV_SIBLINGS_RANGE_HIGH_ = 0x7fffffff
} specv_sibling_rule;

/*
 * specv_accept_resample with the sibling rule given explicitly; the other
 * arguments, outputs and errors are those of specv_accept_resample, except
 * that draft_logits may also be NULL for SPECV_SIBLINGS_DETERMINISTIC, and
 * SPECV_ERR_INVALID_ARG is returned for a rule outside the enum.  At T == 0
 * the rule does not matter (greedy).
 */
specv_status specv_accept_resample_rule(const void* target_logits, const void* draft_logits,
                                        specv_dtype logits_dtype,
                                        const int32_t* tokens, const int32_t* parent,
                                        int32_t B, int32_t K, int32_t V, float temperature,
                                        specv_sibling_rule rule, uint64_t seed, uint64_t offset,
                                        int32_t* accept_len, int32_t* out_tokens, int32_t* out_nodes,
                                        float* p_tok, float* q_tok,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * specv_accept_resample_rule without a workspace argument, for callers that
 * cannot allocate device memory (code under graph capture, tight serving
 * loops, harnesses that forbid allocation).  It allocates nothing: the
 * workspace is an 8 MiB array built into the library, one per device, zero
 * when the library is loaded and kept valid by these calls; it persists until
 * the process ends.  Arguments, outputs and errors are those of
 * specv_accept_resample_rule, except SPECV_ERR_WORKSPACE when the call needs
 * more than 8 MiB of workspace (specv_accept_workspace_bytes; e.g. B = 64,
 * K = 8, V = 151936 in fp32 needs about 0.8 MiB).  Calls that overlap on one
 * device (two streams, two threads without ordering) race on the array and
 * must not be made; calls ordered on one stream are safe.
 */
specv_status specv_accept_resample_rule_noalloc(const void* target_logits, const void* draft_logits,
                                                specv_dtype logits_dtype,
                                                const int32_t* tokens, const int32_t* parent,
                                                int32_t B, int32_t K, int32_t V, float temperature,
                                                specv_sibling_rule rule, uint64_t seed, uint64_t offset,
                                                int32_t* accept_len, int32_t* out_tokens, int32_t* out_nodes,
                                                float* p_tok, float* q_tok, hipStream_t stream);

/*
 * KV-cache commit after a verify step: keep the accepted path, drop the rest.
 *
 * [SD-review] §4 (limitations): the cache entries of rejected drafts have to
 * be rolled back; [SD-EAGLE] "Tree Attention Verification": the verify pass
 * wrote one extra KV-cache entry per tree node, node j's at ctx_len[b] + j.
 * With the accept rule's result (accept_len[b] = a, out_nodes[b] = n_1 < ...
 * < n_a, n_d the accepted node at depth d), the committed sequence is the
 * context, the root and that path: for d = 1 .. a the K and V rows at
 * ctx_len[b] + n_d move to ctx_len[b] + d (rows already in place, n_d == d,
 * are not touched), and the new context length is ctx_len[b] + 1 + a.  Rows
 * at and after the new length are left unspecified (the next verify step
 * writes its tree there).
 *
 *   k_cache, v_cache  [B][Hkv][Lmax][D] dtype, updated in place; 16-byte aligned
 *   ctx_len           [B] int32: context length before the verify step
 *   accept_len        [B] int32, out_nodes [B][K+1] int32: from
 *                     specv_accept_resample on the same tree
 *   dtype             SPECV_BF16 or SPECV_F32 (the cache's element type)
 *   new_ctx_len       [B] int32: ctx_len + 1 + accept_len; -1 (and the
 *                     sequence's cache untouched) if accept_len is outside
 *                     [0, K], ctx_len < 0 or ctx_len + K + 1 > Lmax, or
 *                     out_nodes[0 .. a-1] is not an increasing list with the
 *                     depth-d entry in [d, K]
 *
 * Ownership: device memory owned by the caller; asynchronous on `stream`.
 * Errors: SPECV_ERR_INVALID_ARG (NULL pointer, B < 0, K < 0,
 * K + 1 > SPECV_MAX_NODES, Hkv <= 0, Lmax < K + 1, misaligned cache),
 * SPECV_ERR_UNSUPPORTED (D not 64 or 128, unknown dtype), SPECV_ERR_HIP.
 */
specv_status specv_kv_commit(void* k_cache, void* v_cache, const int32_t* ctx_len,
                             const int32_t* accept_len, const int32_t* out_nodes,
                             int32_t B, int32_t K, int32_t Hkv, int32_t D, int32_t Lmax,
                             specv_dtype dtype, int32_t* new_ctx_len, hipStream_t stream);

/*
 * One level of draft-tree expansion (EAGLE-style top-k children, kept by
 * cumulative draft probability).
 *
 * [SD-EAGLE] "EAGLE: tree drafting and feature reuse": the draft outputs K
 * candidates per depth (exercise 4: the top 3 branches at every depth), and
 * EAGLE-2 grows the tree wide where the draft is unsure, narrow where it is
 * confident; [PTD] Method 2, "Progressive Expansion & Pruning": each step
 * drafts children for all current leaves in one pass, width control caps the
 * children per parent.  For each sequence b:
 *   - every frontier row f whose node u = frontier[b][f] is a node of the tree
 *     (0 <= u < n_nodes[b]) proposes the min(k, V) tokens of largest draft
 *     logit (ties: lower token id), child score = score[u] + log q(token),
 *     q = softmax(draft_logits[b][f] / T);
 *   - of all candidates, the `keep` of highest score survive (ties: earlier
 *     row, then better rank), fewer when the tree reaches nmax nodes;
 *   - survivors are appended as nodes n_nodes[b], n_nodes[b] + 1, ... in row
 *     order, then rank order (parent, token and score written), n_nodes[b]
 *     grows by their number, and their ids go to new_frontier[b] (then -1).
 * Node ids stay topological, so parent[b][0 .. n_nodes) is a valid parent
 * array for specv_build_tree_mask; the tokens of a tree built this way are
 * fixed candidates (SPECV_SIBLINGS_DETERMINISTIC).
 *
 *   draft_logits  [B][F][V] dtype; row f belongs to frontier[b][f]
 *   frontier      [B][F] int32 (entries that are not nodes: no row)
 *   k             children per frontier node, 1 .. SPECV_EXPAND_MAX_K;
 *                 F * k <= SPECV_EXPAND_MAX_CANDIDATES
 *   temperature   T > 0, finite (only the scores depend on it)
 *   keep          survivors per sequence at most, 1 .. SPECV_MAX_NODES (fewer
 *                 when there are fewer candidates)
 *   nmax          capacity of the tree arrays, <= SPECV_MAX_NODES
 *   parent, tokens [B][nmax] int32; score [B][nmax] float64 (cumulative
 *                 draft log-probability; the root's is usually 0); n_nodes [B]
 *                 int32; all read and updated in place
 *   new_frontier  [B][keep] int32
 *   workspace / workspace_bytes: at least specv_tree_expand_workspace_bytes(B, F)
 *
 * Errors: SPECV_ERR_INVALID_ARG (NULL pointer, sizes out of range, T <= 0),
 * SPECV_ERR_UNSUPPORTED (dtype), SPECV_ERR_WORKSPACE, SPECV_ERR_HIP.
 */
#define SPECV_EXPAND_MAX_K 16
#define SPECV_EXPAND_MAX_CANDIDATES 1024

specv_status specv_tree_expand(const void* draft_logits, specv_dtype dtype, const int32_t* frontier,
                               int32_t B, int32_t F, int32_t V, int32_t k, float temperature,
                               int32_t keep, int32_t nmax, int32_t* parent, int32_t* tokens,
                               double* score, int32_t* n_nodes, int32_t* new_frontier,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

size_t specv_tree_expand_workspace_bytes(int32_t B, int32_t F);

/*
 * One target-model layer over the draft nodes (bf16).
 *
 * [SD-EAGLE] "Two-Model Setup" step 2: the target runs one forward pass over
 * all K + 1 positions at once; [PTD] Method 4, "Verification": all tree nodes
 * are verified in one pass that uses the tree mask and the matching position
 * encoding.  The pages name no architecture; this is a pre-norm decoder layer
 * of the common open-model shape, with T = B (K + 1) rows (b, node):
 *   h   = x / sqrt(mean(x^2) + eps) * attn_norm
 *   q, k, v = split(h w_qkv^T)                 (Hq, Hkv, Hkv heads of D)
 *   q, k rotated at position ctx_len[b] + depth[b][i]: the pair (j, j + D/2)
 *        of a head turns by pos * theta^(-2j/D)
 *   k, v written to the caches at ctx_len[b] + i
 *   a   = specv_tree_attn_verify(q, caches, ctx_len, mask)   (scale 1/sqrt(D))
 *   y   = x + a w_o^T
 *   g, u = split(rms(y) * mlp_norm  w_gate_up^T)
 *   out = y + (silu(g) * u) w_down^T
 * Activations are stored in bf16 between the steps; products and norms
 * accumulate in fp32; the rotation angle is formed in fp64.
 *
 *   x                [B][K+1][Hq*D] bf16 hidden states of the nodes
 *   w_qkv            [(Hq + 2 Hkv) D][Hq D]: query rows, then key, then value
 *   w_o              [Hq D][Hq D]
 *   w_gate_up        [2 inter][Hq D]: gate rows, then up rows
 *   w_down           [Hq D][inter]
 *   attn_norm, mlp_norm  [Hq D] gains
 *   rms_eps > 0, rope_theta > 1
 *   k_cache, v_cache [B][Hkv][Lmax][D] bf16: context rows read, the nodes'
 *                    rows [ctx_len, ctx_len + K + 1) written
 *   ctx_len          [B] int32
 *   mask, depth      from specv_build_tree_mask on the same parent array
 *   inter            MLP width, a multiple of 64
 *   out              [B][K+1][Hq*D] bf16; may be x itself
 *   workspace        specv_verify_layer_workspace_bytes(...) bytes, 256-byte
 *                    aligned
 * A sequence with ctx_len < 0, ctx_len + K + 1 > Lmax or an invalid tree
 * (depth -1) gets NaN outputs and its cache is not written.
 *
 * Ownership: device memory owned by the caller; asynchronous on `stream`;
 * every pointer 16-byte aligned.
 * Errors: SPECV_ERR_INVALID_ARG (NULL pointer, B < 0, K < 0,
 * K + 1 > SPECV_MAX_NODES, Hq not a positive multiple of Hkv, Lmax < K + 1,
 * inter not a positive multiple of 64, eps or theta out of range, misaligned
 * pointer), SPECV_ERR_UNSUPPORTED (D not 64 or 128), SPECV_ERR_WORKSPACE,
 * SPECV_ERR_HIP.
 */
specv_status specv_verify_layer(const void* x, const void* w_qkv, const void* w_o,
                                const void* w_gate_up, const void* w_down,
                                const void* attn_norm, const void* mlp_norm,
                                float rms_eps, float rope_theta,
                                void* k_cache, void* v_cache, const int32_t* ctx_len,
                                const uint32_t* mask, const int32_t* depth,
                                int32_t B, int32_t K, int32_t Hq, int32_t Hkv, int32_t D,
                                int32_t Lmax, int32_t inter, void* out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes of specv_verify_layer (0 for invalid sizes). */
size_t specv_verify_layer_workspace_bytes(int32_t B, int32_t K, int32_t Hq, int32_t Hkv, int32_t D,
                                          int32_t Lmax, int32_t inter);

/*
 * A weight matrix of the layer in the tile order its products read (the same
 * layer as specv_verify_layer, [SD-EAGLE] "Two-Model Setup" step 2; the order
 * is a storage format only, the arithmetic is unchanged).
 *
 *   w       [N][K] bf16, row-major ([out][in] of the linear map)
 *   N, K    N a positive multiple of 32, K a positive multiple of 64 (true of
 *           every matrix of the layer: (Hq + 2 Hkv) D, Hq D, 2 inter rows)
 *   packed  N K bf16 elements: 16-byte unit ((rb (K/64) + s) 4 + j) 64 + l
 *           holds w[32 rb + l % 32][64 s + 32 (l / 32) + 8 j .. + 8], so that
 *           each weight load of the product reads 1 KB contiguous
 *
 * Pack once per matrix (weights are static); the gate/up matrix packs as one
 * [2 inter][Hq D] matrix.  Ownership: device memory of the caller, both
 * 16-byte aligned and not overlapping; asynchronous on `stream`.
 * Errors: SPECV_ERR_INVALID_ARG (sizes, NULL, alignment, overlap), SPECV_ERR_HIP.
 */
specv_status specv_pack_weights(const void* w, int32_t N, int32_t K, void* packed, hipStream_t stream);

/*
 * specv_verify_layer with w_qkv, w_o, w_gate_up and w_down each in the order of
 * specv_pack_weights.  Arguments, outputs, workspace and errors are those of
 * specv_verify_layer; the outputs are bit-identical to it (the same products
 * in the same order, only the weights' storage order differs).
 */
specv_status specv_verify_layer_packed(const void* x, const void* w_qkv, const void* w_o,
                                       const void* w_gate_up, const void* w_down,
                                       const void* attn_norm, const void* mlp_norm,
                                       float rms_eps, float rope_theta,
                                       void* k_cache, void* v_cache, const int32_t* ctx_len,
                                       const uint32_t* mask, const int32_t* depth,
                                       int32_t B, int32_t K, int32_t Hq, int32_t Hkv, int32_t D,
                                       int32_t Lmax, int32_t inter, void* out,
                                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Static description of a status code. */
const char* specv_status_string(specv_status s);

/* Text of the last error returned to the calling thread ("" if none). */
const char* specv_last_error(void);

/*
 * Measurement aid, for benchmarks (not part of the method): the streaming-read
 * ceiling that the HBM-bound kernels are compared with.  Reads `bytes` of
 * device memory at `buf` once, with the 16-byte non-temporal loads the
 * statistics and attention streams use, each of a fixed set of workgroups
 * taking one contiguous slice; each workgroup stores one word (a fold of what
 * it read) to sink, so the reads cannot be optimised away.
 *   buf         device, 16-byte aligned, `bytes` a multiple of 16 (0: no-op)
 *   sink        device uint32[sink_words], sink_words >= specv_read_probe_sink_words()
 * Asynchronous on `stream`; time it with events on that stream.  Returns
 * SPECV_ERR_INVALID_ARG (NULL pointer, misalignment, sink too small) or
 * SPECV_ERR_HIP.
 */
specv_status specv_read_probe(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words,
                              hipStream_t stream);
int32_t specv_read_probe_sink_words(void);

/*
 * Debugging aid, for tests (not part of the method): the bounds record of a
 * bounds-checked build of this library (libspecv_checked.so, compiled with
 * SPECV_CHECKED).  In that build every kernel access whose index is derived
 * from input data (parent and token values, context lengths, accepted node
 * ids, frontier entries) is checked against its range; the first index out
 * of range is recorded (site number in bits 32-63, the index in bits 0-31)
 * and replaced by 0, so the access stays in its buffer.
 *   reset  nonzero: clear the record after reading it
 * Returns 0 if nothing was recorded, the record otherwise, and -1 in the
 * product build (no checks compiled in).  Synchronises the current device
 * first (in the checked build); -2 if that or the read fails.
 */
int64_t specv_debug_bounds(int32_t reset);

#ifdef __cplusplus
}
#endif

#endif /* SPECV_H */
