/*
 * sv.h -- draft-tree verification on AMD Instinct MI355X (gfx950): C ABI.
 *
 * One verification step of EAGLE-style speculative decoding, as described on
 *   [EAGLE article]  the course.zhidx.com mirror of the Zhihu article on
 *                    EAGLE / EAGLE-2 / EAGLE-3 / DFlash: section 1.3
 *                    "Verification" (one target forward scores the whole draft
 *                    tree with tree attention; speculative sampling is applied
 *                    recursively at every node, with k sibling candidates tried
 *                    in turn, Figure 1-6) and section 2.3 "Flatten + Attention
 *                    mask" (each token sees only its ancestors, Figure 2-7);
 *   [Spec-decoding lesson]  "Speculative decoding and EAGLE"
 *                    (ai-engineering.com.cn): sections "Concept" (K+1 positions,
 *                    bonus token), "Exactness rule" (accept iff r < p(x)/q(x),
 *                    else sample (p-q)+ normalised; greedy: accept iff
 *                    argmax(p) == x) and "Tree-attention verification".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All array arguments are DEVICE pointers owned by the caller (any device
 *    allocator).  Structs are HOST structs, read during the call and not kept.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Every call only enqueues work on that stream: it never allocates, frees
 *    or synchronises, and returns as soon as the work is queued.
 *  - Return value: SV_OK (0) or a negative sv_status.  Problems visible from
 *    the host (null pointers, bad sizes, a workspace that is too small,
 *    unsupported shapes) are reported before anything is launched; a launch
 *    failure returns SV_E_HIP.  sv_last_error() gives a detail string for the
 *    calling thread.  Calls may come from several host threads at once; the
 *    library's only shared host state is a per-device cache of occupancy and
 *    device facts, filled with atomic stores.
 *  - Problems in the data (a malformed tree, a token outside the vocabulary,
 *    a non-finite target logit) are per sequence: they are reported on the
 *    device in tree_status[b] (SV_TREE_*), and that sequence's outputs are
 *    written as zeros / -1 / count 0.  Other sequences are unaffected.
 *  - Flattened trees: position 0 of every sequence is the root (the last
 *    emitted token, verified in the same pass); positions 1..T_b-1 are the
 *    draft nodes in an order where every parent precedes its children
 *    (parent[i] < i).  Siblings are tried in increasing position, which must
 *    be the order the drafter drew them in.
 *  - Limits: 1 <= T_max <= 256; D in {64, 128}; Hq % Hkv == 0; V >= 1.
 */
#ifndef SV_H_
#define SV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t sv_status;

/* Host-side return codes. */
enum {
  SV_OK = 0,
  SV_E_NULL = -1,        /* a required pointer is NULL                              */
  SV_E_SHAPE = -2,       /* a size is out of range or inconsistent                  */
  SV_E_DTYPE = -3,       /* unknown dtype code                                      */
  SV_E_WORKSPACE = -4,   /* ws_bytes < sv_workspace_bytes(...) or ws misaligned     */
  SV_E_HIP = -5,         /* a HIP runtime call or kernel launch failed              */
  SV_E_UNSUPPORTED = -6  /* valid but not supported (T_max > 256, D not 64/128, ...) */
};

/* Per-sequence device-side status (tree_status[b]). */
enum {
  SV_TREE_OK = 0,
  SV_TREE_E_ROOT = 1,      /* parent[b][0] != -1                                      */
  SV_TREE_E_PARENT = 2,    /* some 1 <= i < T_b has parent[b][i] outside [0, i)       */
  SV_TREE_E_COUNT = 3,     /* num_nodes[b] outside [1, T_max]                         */
  SV_TREE_E_TOKEN = 4,     /* a draft token tokens[b][i], 1 <= i < T_b, outside [0, V) */
  SV_TREE_E_NONFINITE = 5, /* a NaN or +-Inf in the logits row of a node the walk visits */
  SV_TREE_E_NOQ = 6,       /* temperature[b] > 0 but q_probs is NULL                  */
  SV_TREE_E_SYNC = 7,      /* a cross-workgroup wait of the walk timed out (see
                              sv_spec_accept); outputs -1 / count 0                    */
  SV_TREE_E_CACHE = 8,     /* commit: L_b + out_count[b] exceeds L_max (or L_b < 0)   */
  SV_TREE_E_PATH = 9,      /* commit: out_count[b] > T_b or a path entry outside [1, T_b) */
  SV_TREE_E_PROB = 10      /* tree builder: a draft probability outside [0, 1] or NaN  */
};

/* Element types. */
enum { SV_F32 = 0, SV_BF16 = 1 };

/* How the siblings of one node were drafted (decides the proposal each of
 * them is tested against, see sv_spec_accept). */
enum { SV_SIB_WITHOUT_REPLACEMENT = 0, SV_SIB_IID = 1 };

/* Flattened draft trees of a batch. */
typedef struct {
  int32_t B;                /* sequences, >= 0                                        */
  int32_t T_max;            /* padded positions per sequence (root + draft nodes)     */
  const int32_t* parent;    /* [B][T_max]; parent[b][0] = -1, 0 <= parent[b][i] < i   */
  const int32_t* num_nodes; /* [B]; T_b = root + draft nodes, 1 <= T_b <= T_max       */
  const int32_t* tokens;    /* [B][T_max]; token of each position; the root's (position
                               0) is never read, draft tokens must be in [0, V)       */
} sv_tree;

/* Tree attention inputs (post-RoPE projections of one layer). */
typedef struct {
  int32_t Hq, Hkv, D;       /* query heads, KV heads (Hq % Hkv == 0), head dim          */
  int32_t L_max;            /* capacity of the cache's length axis (>= max L_b);        */
                            /* (L_max + 256) * D < 2^31, else SV_E_UNSUPPORTED          */
  int32_t dtype;            /* SV_F32 or SV_BF16, for q, k_new, v_new, caches and out   */
  float scale;              /* score scale; <= 0 means 1/sqrt(D)                        */
  const void* q;            /* [B][T_max][Hq][D]  queries of the tree positions         */
  const void* k_new;        /* [B][T_max][Hkv][D] keys of the tree positions            */
  const void* v_new;        /* [B][T_max][Hkv][D] values of the tree positions          */
  const void* k_cache;      /* [B][Hkv][L_max][D] prefix keys (read only)               */
  const void* v_cache;      /* [B][Hkv][L_max][D] prefix values (read only)             */
  const int32_t* prefix_len;/* [B]; L_b in [0, L_max] (a sequence outside: zero output)   */
  void* out;                /* [B][T_max][Hq][D]; rows i >= T_b written as 0            */
} sv_attn_args;

/* Accept / reject inputs and outputs. */
typedef struct {
  int32_t V;                 /* vocabulary size                                          */
  int32_t logit_dtype;       /* SV_F32 or SV_BF16 for target_logits                      */
  int32_t sibling_mode;      /* SV_SIB_WITHOUT_REPLACEMENT or SV_SIB_IID                 */
  const void* target_logits; /* [B][T_max][V]; row n = target logits for the token
                                following position n                                      */
  const float* q_probs;      /* [B][T_max][V]; row n = draft distribution n's children
                                were drawn from (already at temperature).  May be NULL
                                when every temperature is 0.                              */
  const float* temperature;  /* [B]; 0 selects greedy verification for that sequence     */
  const float* u_accept;     /* [B][T_max] in [0,1): uniform for testing candidate i     */
  const float* u_sample;     /* [B][T_max] in [0,1): uniform for the draw at terminal n  */
  int32_t* out_tokens;       /* [B][T_max]; accepted tokens then the drawn one, -1 pad   */
  int32_t* out_nodes;        /* [B][T_max]; accepted positions (root excluded), -1 pad   */
  int32_t* out_count;        /* [B]; accepted + 1 (0 for an invalid sequence)            */
  int32_t* out_passes;       /* [B] or NULL: vocabulary passes the walk made             */
} sv_accept_args;

/* Ancestor-or-self mask of every tree, plus node depths and the validity of
 * each tree ([EAGLE article] sec. 2.3 "Flatten + Attention mask";
 * [Spec-decoding lesson] "Tree-attention verification").
 *   anc         [B][T_max][W] uint64, W = ceil(T_max / 64): bit (j % 64) of
 *               word j / 64 of row i is set iff j == i or j is an ancestor of i.
 *               Rows and bits >= T_b, and all rows of an invalid tree, are 0.
 *   depth       [B][T_max] int32: edges from the root (0 for padding/invalid).
 *   tree_status [B] int32: SV_TREE_OK, _ROOT, _PARENT or _COUNT (written).
 * Needs no workspace. */
sv_status sv_tree_mask_build(const sv_tree* tree, uint64_t* anc, int32_t* depth,
                             int32_t* tree_status, void* stream);

/* Tree attention ([EAGLE article] sec. 1.3 "Verification";
 * [Spec-decoding lesson] "Tree-attention verification"): for every sequence b
 * with tree_status[b] == 0, position i < T_b and query head h, attend with
 * softmax(scale * q.k) over the first L_b cache entries of KV head
 * h / (Hq / Hkv) and over the tree positions j whose bit is set in anc[b][i].
 * Accumulation is fp32; out is written in `dtype`.  Rows of invalid sequences
 * and rows i >= T_b are written as zeros.
 *   anc, tree_status: as produced by sv_tree_mask_build (read only).
 *   ws / ws_bytes: device workspace of at least sv_workspace_bytes(tree, a, NULL)
 *   bytes, 256-byte aligned (may be NULL when that size is 0). */
sv_status sv_tree_attn(const sv_tree* tree, const uint64_t* anc, const int32_t* tree_status,
                       const sv_attn_args* a, void* ws, size_t ws_bytes, void* stream);

/* Speculative accept / reject over each tree ([Spec-decoding lesson]
 * "Exactness rule", "Concept"; [EAGLE article] sec. 1.3, Figure 1-6).
 * For sequence b (tree_status[b] == 0 on entry), starting at the root:
 *   - p_n = softmax(target_logits[b][n] / temperature[b]) (float32 on device);
 *   - greedy (temperature 0): the first child whose token equals
 *     argmax(target_logits[b][n]) (lowest index on ties) is accepted and the
 *     walk continues there; otherwise argmax is emitted and the walk stops;
 *   - stochastic: children are tested in increasing position.  Candidate c
 *     with token x is accepted iff u_accept[b][c] < P(x) / q_c(x), where P is
 *     the current target (p_n, then the normalised residual) and q_c is the
 *     proposal x was drawn from: q_n with the earlier siblings' tokens removed
 *     and renormalised (SV_SIB_WITHOUT_REPLACEMENT) or q_n itself (SV_SIB_IID).
 *     On rejection P becomes max(0, P - q_c) normalised.  When all children
 *     are rejected, or n is a leaf (bonus token, P = p_n), the emitted token is
 *     the smallest v with sum_{w<=v} P(w) > u_sample[b][n].
 * Outputs: out_nodes = accepted positions, out_tokens = their tokens followed
 * by the emitted token, out_count = accepted + 1.  tree_status[b] may be set to
 * SV_TREE_E_TOKEN, _NONFINITE, _NOQ or _SYNC (then outputs are -1 / count 0).
 * Only the logits rows of the nodes the walk visits (the root and the accepted
 * nodes) are read, and only those are checked for NaN / infinity; draft rows
 * are read for the visited nodes with a rejection.
 *   ws / ws_bytes: at least sv_workspace_bytes(tree, NULL, a) bytes, 256-byte
 *   aligned.  The walk kernel's workgroups (at most one per CU) wait for one
 *   another, so all of them must be resident together: on a device shared with
 *   other work, workgroups queued behind it start when it ends.  A wait longer
 *   than 2 s gives up: the sequence being walked, and every later sequence the
 *   same workgroup group would have walked, get SV_TREE_E_SYNC (a sequence
 *   with its own data error keeps that status) and -1 / count 0 outputs, and
 *   every workgroup ends.  Sequences finished before that keep their results.
 *   (One workgroup of each group writes all of its sequences' outputs.)  Two walks that overlap on one device
 *   (calls on different streams) can each take part of the CUs the other's
 *   groups need, and then both end with SV_TREE_E_SYNC: order walks on one
 *   device (one stream, or events between streams).  Returns
 *   SV_E_UNSUPPORTED if the grid cannot be resident at once. */
sv_status sv_spec_accept(const sv_tree* tree, int32_t* tree_status, const sv_accept_args* a,
                         void* ws, size_t ws_bytes, void* stream);

/* One verification step: sv_tree_mask_build, then sv_tree_attn, then
 * sv_spec_accept, in stream order, sharing one workspace of at least
 * sv_workspace_bytes(tree, attn, acc) bytes: the attention's partial results
 * first, then the accept's exchange words, which the mask kernel zeroes (so
 * the step launches three kernels).  Results are those of the three calls
 * made one after another; the walk's rule on overlapping calls applies to
 * steps too. */
sv_status sv_verify_step(const sv_tree* tree, const sv_attn_args* attn, const sv_accept_args* acc,
                         uint64_t* anc, int32_t* depth, int32_t* tree_status, void* ws,
                         size_t ws_bytes, void* stream);

/* sv_verify_step without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The step's scratch memory (the
 * attention's partial results and the walk's exchange words, the same layout
 * sv_verify_step puts in its workspace) lives in one array per device inside
 * the library, 64 MiB (67108864 bytes), made when the library's code is
 * loaded on that device and kept until the process ends.  The first call on
 * a device looks up that device's array address once.  The call allocates
 * and frees nothing, and the mask kernel zeroes what must start at zero, so
 * results equal those of sv_verify_step.  Every call on one device shares
 * that device's array: calls that overlap on one device (different streams,
 * or host threads without ordering) race on it and must be ordered by the
 * caller.  Returns SV_E_WORKSPACE, before launching anything, when the
 * problem needs more than 64 MiB (sv_workspace_bytes(tree, attn, acc) >
 * 67108864); other errors as sv_verify_step. */
sv_status sv_verify_step_noalloc(const sv_tree* tree, const sv_attn_args* attn, const sv_accept_args* acc,
                                 uint64_t* anc, int32_t* depth, int32_t* tree_status, void* stream);

/* Commit of the accepted path: cache growth and drafter features. */
typedef struct {
  int32_t Hkv, D;           /* KV heads and head dim of the caches (any D with D*size % 16 == 0) */
  int32_t L_max;            /* capacity of the caches' length axis                      */
  int32_t dtype;            /* SV_F32 or SV_BF16 for k_new, v_new and the caches        */
  const void* k_new;        /* [B][T_max][Hkv][D] keys of the verified positions        */
  const void* v_new;        /* [B][T_max][Hkv][D] values of the verified positions      */
  void* k_cache;            /* [B][Hkv][L_max][D]: rows [L_b, L_b + c) written          */
  void* v_cache;            /* [B][Hkv][L_max][D]: rows [L_b, L_b + c) written          */
  const int32_t* prefix_len;/* [B] L_b before the commit (read)                         */
  int32_t* prefix_len_out;  /* [B] L_b + c (L_b when nothing is committed); must not
                               alias prefix_len                                          */
  int32_t F;                /* feature width per position; 0 = no features              */
  int32_t feat_dtype;       /* SV_F32 or SV_BF16 for feat_in / feat_out                 */
  const void* feat_in;      /* [B][T_max][F] features of the verified positions         */
  void* feat_out;           /* [B][T_max][F]: rows [0, c) = committed positions' rows,
                               other rows zero                                           */
} sv_commit_args;

/* Commit of the accepted path ([EAGLE article] sec. 1.3 "Verification": the
 * accepted tokens and their features are kept and drafting continues from
 * them; [Spec-decoding lesson] "Concept": the accepted tokens extend the
 * output and the correction / bonus token is the next position to run).
 * For every sequence b with tree_status[b] == 0 and c = out_count[b] >= 1,
 * the verified positions [0 (root), out_nodes[b][0], ..., out_nodes[b][c-2]]
 * have their K and V rows (every KV head) copied, bit for bit, to cache rows
 * L_b .. L_b + c - 1, prefix_len_out[b] = L_b + c, and their feature rows to
 * feat_out rows 0 .. c-1.  The emitted token out_tokens[b][c-1] is the next
 * root: its rows come from the next forward pass.
 *   tree: B, T_max, num_nodes (parent and tokens are not read).
 *   tree_status [B] (in/out): sequences not OK are left alone; SV_TREE_E_CACHE
 *   or SV_TREE_E_PATH is written when a commit does not fit or the path is out
 *   of range (then nothing of that sequence is written, prefix_len_out = L_b).
 *   out_nodes / out_count: as written by sv_spec_accept.
 * Needs no workspace.  Tensors must be 16-byte aligned. */
sv_status sv_commit_accepted(const sv_tree* tree, int32_t* tree_status, const int32_t* out_nodes,
                             const int32_t* out_count, const sv_commit_args* c, void* stream);

/* ---------------------------------------------------------------- tree builder
 * EAGLE-2 draft-tree construction ([EAGLE article] sec. 2.3 "Context-aware
 * draft tree"; sec. 2.2 for draft confidence as the acceptance estimate).
 * A node's value is the product of the draft probabilities along its path
 * from the root (value 1).  Each step expands the k best nodes of the newest
 * layer ("Expansion Phase"): the drafter's probability row of each such node
 * gives it k children, its k most probable tokens (probability descending,
 * ties to the lower token id).  After the last step the m best draft nodes
 * over the whole tree are kept ("Reranking Phase": value descending, equal
 * values to the shallower node, then to the earlier created), which is a
 * connected tree because a child's value never exceeds its parent's, and the
 * kept tree is flattened for verification: by depth, then parent position,
 * then sibling rank, so parents precede children (the parent array that
 * sv_tree_mask_build takes).  Values are float32 products, one IEEE multiply
 * per node; every selection compares them exactly.
 *
 * Use: sv_eagle2_begin, then for step = 0 .. depth-1 run the drafter on the
 * current frontier (the root at step 0) and call sv_eagle2_expand with its
 * probability rows, then sv_eagle2_finish (or, for the last step,
 * sv_eagle2_expand_finish, which does both).  All calls only enqueue work on the
 * stream; the state lives in one caller buffer of sv_eagle2_state_bytes bytes
 * (256-byte aligned), and calls on one state must be in this order. */
typedef struct {
  int32_t B;       /* sequences                                                      */
  int32_t V;       /* vocabulary size (k <= V <= 524288)                                */
  int32_t k;       /* expansion width: nodes expanded per step and children per node, 1..16 */
  int32_t depth;   /* expansion steps, >= 1                                           */
  int32_t m;       /* draft nodes kept, 1 <= m <= k + (depth-1) k^2 and m + 1 <= 256;
                      the tree has k + (depth-1) k^2 + 1 <= 2048 nodes before the rerank */
} sv_eagle2_cfg;

/* State bytes for a configuration (host only); 0 if it is invalid or
 * unsupported (see sv_last_error). */
size_t sv_eagle2_state_bytes(const sv_eagle2_cfg* c);

/* Starts the trees: node 0 of sequence b is root_tokens[b] (device [B] int32)
 * with value 1; the frontier is the root. */
sv_status sv_eagle2_begin(const sv_eagle2_cfg* c, void* state, size_t state_bytes,
                          const int32_t* root_tokens, void* stream);

/* One expansion step.  q (device, float32 [B][k][V], 16-byte aligned): row j
 * of sequence b is the drafter's probability row for frontier entry j.  Step
 * 0 reads row 0 (the root's) only; later steps read all k rows of every
 * sequence (the frontier is full then), and a sequence that has failed
 * ignores what it read.
 * Every row that is read is checked: a value outside [0, 1] or NaN sets the
 * sequence's status to SV_TREE_E_PROB and its later steps do nothing.
 * frontier (device int32 [B][k], may be NULL): the node ids of the next
 * frontier, -1 padded; frontier_tokens (device int32 [B][k], may be NULL):
 * their tokens, -1 padded.  step must count 0, 1, ..., depth-1. */
sv_status sv_eagle2_expand(const sv_eagle2_cfg* c, void* state, size_t state_bytes, int32_t step,
                           const float* q, int32_t* frontier, int32_t* frontier_tokens, void* stream);

/* The rerank and flattening.  Outputs (device, int32): parent, tokens, q_row
 * [B][m+1] and num_nodes, status [B].  Position 0 is the root (parent -1).
 * q_row[b][i] = step * k + j when the node at position i was frontier entry j
 * of that step (its draft probabilities are row j of that step's q), else -1.
 * A sequence with status SV_TREE_E_PROB gets num_nodes 0 and -1 elsewhere. */
sv_status sv_eagle2_finish(const sv_eagle2_cfg* c, const void* state, size_t state_bytes,
                           int32_t* parent, int32_t* tokens, int32_t* num_nodes, int32_t* q_row,
                           int32_t* status, void* stream);

/* sv_eagle2_expand followed by sv_eagle2_finish, with the same arguments and
 * results, in one launch after the row top-k: the workgroup that appends a
 * sequence's last layer also reranks and flattens its tree, so the finish
 * needs no launch and no second read of the state.  Meant for the last step
 * (step = depth - 1); the next frontier is not written.  Same errors as the
 * two calls (checked before anything is enqueued). */
sv_status sv_eagle2_expand_finish(const sv_eagle2_cfg* c, void* state, size_t state_bytes, int32_t step,
                                  const float* q, int32_t* parent, int32_t* tokens, int32_t* num_nodes,
                                  int32_t* q_row, int32_t* status, void* stream);

/* ---------------------------------------------------------------- draft head
 * Two-stage draft LM head ([EAGLE-4 blog], sections "EAGLE Efficient LM
 * Head", "A training-free version: Freq-aware SVD", "A variant based on Local
 * Top-k").  Stage 1: u = B h.  Stage 2: approximate scores A u over a
 * shuffled vocabulary, and in each tile of `tile` consecutive shuffled rows
 * the k_tile best per position are kept as candidates (the scores never leave
 * the chip).  Stage 3: exact logits W[id] . h for the candidates only.  A and
 * B are low-rank factors of W made offline (for example the page's
 * frequency-weighted truncated SVD, A = F^(-1/2) U_r S_r, B = V_r^T with
 * F^(1/2) W = U S V^T); A's rows are stored in the shuffled order and perm
 * maps a shuffled row to its token id.
 * Precision: bf16 inputs, float32 accumulation; u is stored as bf16 (rounded
 * to nearest even); within a tile, equal scores go to the lower shuffled row.
 * Candidates of position i are cand_ids[i][t * k_tile + c] for tile t and
 * rank c; a last tile shorter than k_tile pads with id -1 and logit 0. */
typedef struct {
  int32_t N;                /* draft positions (rows of h), >= 0                        */
  int32_t d;                /* hidden size, a multiple of 32                            */
  int32_t r;                /* rank of the factors, a multiple of 32, <= 2048           */
  int32_t n;                /* vocabulary size, >= 1                                    */
  int32_t tile;             /* shuffled rows per tile, a multiple of 16 in [16, 256]    */
  int32_t k_tile;           /* candidates kept per tile, 1..8, <= tile                  */
  const void* h;            /* [N][d] bf16 hidden states                                 */
  const void* B;            /* [r][d] bf16                                               */
  const void* A_sh;         /* [n][r] bf16, rows in shuffled order                       */
  const int32_t* perm;      /* [n] token id of each shuffled row                         */
  const void* W;            /* [n][d] bf16 full head, rows in token order                */
  void* u;                  /* [N][r] bf16 out: stage 1                                  */
  int32_t* cand_ids;        /* [N][ceil(n / tile) * k_tile] out: candidate token ids     */
  float* cand_logits;       /* [N][ceil(n / tile) * k_tile] out: their exact logits      */
} sv_head_args;

/* Runs the three stages in stream order; needs no workspace.  All arrays are
 * device memory, 16-byte aligned (h, B, A_sh, W, u).  Inputs are trusted to
 * be finite and perm to be a permutation of [0, n); ids outside [0, n) give
 * logit 0. */
sv_status sv_draft_head(const sv_head_args* a, void* stream);

/* Workspace bytes needed by sv_tree_attn (attn != NULL), sv_spec_accept
 * (acc != NULL) or sv_verify_step (both: the attention's region followed by
 * the accept's, which is enough for either call alone too).  Host only;
 * reads only the scalar fields of the structs.  Returns 0 on invalid sizes
 * (see sv_last_error). */
size_t sv_workspace_bytes(const sv_tree* tree, const sv_attn_args* attn, const sv_accept_args* acc);

/* Static description of a status code (host or tree status). */
const char* sv_status_string(sv_status s);

/* Detail of the last host-side error on the calling thread ("" if none). */
const char* sv_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* SV_H_ */
