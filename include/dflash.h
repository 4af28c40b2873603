/*
 * dflash.h -- C ABI of the MI355X (gfx950) library for one DFlash
 * block-diffusion draft-and-verify step.
 *
 * The step has three parts, one entry point each:
 *
 *   dflash_inject_kv      target features of newly accepted positions, taken
 *                         from several target layers, are fused (fc + RMSNorm)
 *                         and projected into the K/V of every draft layer, then
 *                         appended to the draft KV cache.
 *                         ("DFlash, Diffusion LLMs, dLLM, MTP and Speculative
 *                         Decoding: A Deep Research Report", section "Key
 *                         points": KV injection into every draft layer.)
 *   dflash_draft_forward  one drafting pass over a block of B slots (the last
 *                         accepted token, then B-1 mask tokens), attention
 *                         bidirectional inside the block and over the whole
 *                         injected context, shared lm_head, argmax per slot.
 *                         (Same page, "Key points" and "Why DFlash beats
 *                         EAGLE-3" item 3; "Term: DFlash speculative
 *                         decoding", section "DFlash: architecture and
 *                         workflow", stage two.)
 *   dflash_verify_accept  target lm_head argmax at the B+1 block rows, the
 *                         longest prefix on which the draft matches, and the
 *                         target's token at the first mismatch.
 *                         ("Term: DFlash speculative decoding", "DFlash:
 *                         architecture and workflow", stages three and four.)
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers are DEVICE pointers unless marked [host].  The caller owns all
 *   memory (weights, cache, inputs, outputs, workspace); the library never
 *   allocates or frees.
 * - Every call enqueues work on the given HIP stream and returns without
 *   synchronising.  Host-side validation runs first and is all-or-nothing:
 *   on a negative return nothing was enqueued.  dflash_last_error() gives a
 *   thread-local message for the last failure.
 * - Element type: dims->dtype selects the storage type of weights, features,
 *   target hidden states and the KV cache: DFLASH_BF16 (bfloat16) or
 *   DFLASH_F32.  Accumulation is always fp32; the residual stream is fp32.
 * - Matrices are given to the pack calls in PyTorch Linear layout
 *   [out_features, in_features], row-major.  The step calls take PACKED
 *   matrices (see "Packed layout").
 * - Device-side faults (a KV capacity overflow, a token id outside
 *   [0, vocab)) set sticky bits in kv->status and never fault the GPU.
 * - A workspace must be zero-filled once (dflash_workspace_init) before its
 *   first use.  Calls that share one workspace must run in stream order on
 *   one stream; two calls overlapping on one workspace race.
 *
 * Packed layout ("fragment tiles")
 * --------------------------------
 * A packed matrix of R rows and K columns is a sequence of 1 KiB tiles of 16
 * rows x KT columns (KT = 32 for bf16, 16 for fp32), ordered row-tile major
 * then column tile.  Inside a tile, the 16 bytes at offset 16*l hold row
 * (l % 16) and columns (l / 16) * E .. (l / 16) * E + E - 1 with E = KT / 4.
 * This is the register image of one 64-lane MFMA operand, so a wavefront
 * reads a tile with one fully coalesced 1 KiB load.  Rows and columns beyond
 * R and K are zero.
 */
#ifndef DFLASH_H
#define DFLASH_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DFLASH_ABI_VERSION 1

typedef enum { DFLASH_BF16 = 0, DFLASH_F32 = 1 } dflash_dtype;

typedef enum {
  DFLASH_OK = 0,
  DFLASH_ERR_NULL = -1,        /* a required pointer is NULL */
  DFLASH_ERR_SHAPE = -2,       /* a size or dimension is out of range */
  DFLASH_ERR_DTYPE = -3,       /* unknown dtype */
  DFLASH_ERR_WORKSPACE = -4,   /* workspace too small */
  DFLASH_ERR_ALIGN = -5,       /* a pointer is not 16-byte aligned */
  DFLASH_ERR_HIP = -6,         /* a HIP call or kernel launch failed */
  DFLASH_ERR_UNSUPPORTED = -7  /* well-formed dims outside the kernels' limits */
} dflash_status;

/* Sticky bits OR-ed into *kv->status by device code. */
#define DFLASH_STATUS_CAPACITY 1u  /* an injection would exceed kv->capacity */
#define DFLASH_STATUS_TOKEN 2u     /* a token id outside [0, vocab) was clamped */
#define DFLASH_STATUS_ANCHOR 4u    /* an anchor outside its sequence's cache was clamped */
#define DFLASH_STATUS_TREE 8u      /* a malformed tree parent was read as the previous node */

/* Drafter dimensions [host].  Every call that takes dims checks them first.
 * DFLASH_ERR_SHAPE (malformed): hidden, head_dim, intermediate and vocab
 * must be positive multiples of 32; n_q_heads % n_kv_heads == 0 with both
 * positive; n_layers >= 1; n_feat_layers >= 1; 1 <= block_size <= 16;
 * 0 <= mask_id < vocab; rms_eps >= 0 and rope_theta >= 0.
 * DFLASH_ERR_UNSUPPORTED (well-formed, but outside what the kernels are
 * built for): hidden must be a multiple of 64 and at most 8192; head_dim 64
 * or 128; n_q_heads / n_kv_heads <= 16; n_layers <= 16.
 * rope_theta == 0 turns rotary embedding off. */
typedef struct {
  int32_t hidden;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t n_layers;
  int32_t intermediate;
  int32_t vocab;
  int32_t n_feat_layers;
  int32_t block_size;
  int32_t mask_id;
  float rope_theta;
  float rms_eps;
  int32_t dtype;
} dflash_dims;

/* One draft layer.  Norm gains are plain vectors [hidden] of the storage
 * type; matrices are packed by the dflash_pack_* calls. */
typedef struct {
  const void *attn_norm;  /* [H] */
  const void *w_qkv;      /* dflash_pack_qkv output */
  const void *w_o;        /* dflash_pack_matrix of W_o [H, n_q*d] */
  const void *mlp_norm;   /* [H] */
  const void *w_gate_up;  /* dflash_pack_gate_up output */
  const void *w_down;     /* dflash_pack_matrix of W_down [H, I] */
} dflash_layer;

typedef struct {
  const void *w_fc;        /* dflash_pack_matrix of W_fc [H, n_f*H] */
  const void *fc_norm;     /* [H] */
  const void *embed;       /* plain row-major [V, H] (rows are gathered) */
  const void *final_norm;  /* [H] */
  const void *lm_head;     /* dflash_pack_lm_head of W_lm [V, H] */
  const dflash_layer *layers;  /* [host] array of n_layers */
} dflash_weights;

/* Draft KV cache.  k and v each hold n_layers * max_batch * n_kv_heads
 * regions of `capacity` positions (dflash_kv_bytes each), in the packed
 * cache layout that dflash_kv_import / dflash_kv_export convert from / to the
 * plain layout [n_layers][max_batch][n_kv_heads][capacity][head_dim].
 * ctx_len[s] is the number of valid positions of sequence s. */
typedef struct {
  void *k;
  void *v;
  int32_t *ctx_len;   /* [max_batch] */
  uint32_t *status;   /* one word of sticky DFLASH_STATUS_* bits */
  int32_t capacity;   /* [host] positions per sequence, a multiple of 32 */
  int32_t max_batch;  /* [host] */
} dflash_kv;

/* ---------------------------------------------------------------- packing */

/* Bytes of a packed R x K matrix of the given dtype (rows rounded up to 16,
 * columns to KT). */
size_t dflash_packed_bytes(int32_t dtype, int32_t rows, int32_t cols);

/* Pack a row-major [rows, cols] matrix.  dst must hold
 * dflash_packed_bytes(dtype, rows, cols); src and dst 16-byte aligned. */
int dflash_pack_matrix(int32_t dtype, const void *src, int32_t rows, int32_t cols,
                       void *dst, hipStream_t stream);

/* Pack the q, k and v projections of one layer (W_q [n_q*d, H],
 * W_k / W_v [n_kv*d, H]) into one matrix of (n_q + 2 n_kv) * d rows.  Rows of
 * q and k heads are reordered so that each rotary pair (channels i and
 * i + d/2) shares a 16-row tile; v keeps its order.  dst holds
 * dflash_packed_bytes(dtype, (n_q + 2 n_kv) * d, H). */
int dflash_pack_qkv(const dflash_dims *dims, const void *wq, const void *wk, const void *wv,
                    void *dst, hipStream_t stream);

/* Pack W_gate and W_up ([I, H] each) into one matrix of 2I rows in the
 * paired layout: row tiles alternate gate, up, gate, up..., and each pair of
 * row tiles (2p, 2p + 1) interleaves per column tile, so tile (2p + j, c)
 * sits at position (p * K_tiles + c) * 2 + j.  dst holds
 * dflash_packed_bytes(dtype, 2 * I, H). */
int dflash_pack_gate_up(const dflash_dims *dims, const void *w_gate, const void *w_up,
                        void *dst, hipStream_t stream);

/* Pack the shared lm_head W_lm [vocab, hidden] in the paired layout (row
 * tiles 2p and 2p + 1 interleave per column tile, as for dflash_pack_gate_up)
 * that the draft and verify heads read: a wavefront's K range of two row
 * tiles is then one contiguous run.  vocab a multiple of 32; dst holds
 * dflash_packed_bytes(dtype, vocab, hidden). */
int dflash_pack_lm_head(int32_t dtype, const void *src, int32_t vocab, int32_t hidden, void *dst,
                        hipStream_t stream);

/* --------------------------------------------------------------- KV cache */

/* Bytes of each of kv->k and kv->v. */
size_t dflash_kv_bytes(const dflash_dims *dims, int32_t capacity, int32_t max_batch);

/* Copy a whole cache between the plain layout
 * [n_layers][max_batch][n_kv][capacity][head_dim] (storage dtype) and the
 * packed layout.  ctx_len is neither read nor written. */
int dflash_kv_import(const dflash_dims *dims, const dflash_kv *kv, const void *k_plain,
                     const void *v_plain, hipStream_t stream);
int dflash_kv_export(const dflash_dims *dims, const dflash_kv *kv, void *k_plain,
                     void *v_plain, hipStream_t stream);

/* -------------------------------------------------------------- workspace */

/* Workspace bytes for calls with at most max_batch sequences and at most
 * max_rows injected rows per dflash_inject_kv call. */
size_t dflash_workspace_bytes(const dflash_dims *dims, int32_t max_batch, int32_t max_rows);

/* Zero-fill a workspace (once, after allocation). */
int dflash_workspace_init(void *ws, size_t ws_bytes, hipStream_t stream);

/* Where the last call of a given kind left an intermediate, for checks:
 *   DFLASH_VIEW_FUSED     fp32 [rows, H]: fused target features W_fc f of
 *                         the injected rows, before their RMSNorm
 *   DFLASH_VIEW_HIDDEN    fp32 [batch*B, H]: residual after layer `layer`
 *                         (layer = -1: the block embeddings)
 *   DFLASH_VIEW_MID       fp32 [batch*B, H]: residual after the attention
 *                         half of layer `layer`
 *   DFLASH_VIEW_ATTN      fp32 [batch*B, n_q*d]: attention output of layer
 *                         `layer`, before the output projection
 * `count` is rows for FUSED and batch otherwise.  Offsets are from ws. */
enum {
  DFLASH_VIEW_FUSED = 0,
  DFLASH_VIEW_HIDDEN = 1,
  DFLASH_VIEW_MID = 2,
  DFLASH_VIEW_ATTN = 3
};
int dflash_workspace_view(const dflash_dims *dims, int32_t what, int32_t count, int32_t layer,
                          size_t *offset, size_t *bytes);

/* ------------------------------------------------------------- the step */

/* KV injection.  feats: [rows, n_feat_layers * H] row-major, storage dtype,
 * feature layer k in columns [k H, (k+1) H).  cu_new: [batch + 1] prefix sums
 * of rows per sequence (cu_new[0] = 0, cu_new[batch] = rows).  Row i of
 * sequence s is written at cache position ctx_len[s] + i with rotary
 * position ctx_len[s] + i; then ctx_len[s] += n_s.  A sequence whose new
 * length would exceed kv->capacity is skipped whole and sets
 * DFLASH_STATUS_CAPACITY.  rows [host] must equal cu_new[batch]. */
int dflash_inject_kv(const dflash_dims *dims, const dflash_weights *w, const dflash_kv *kv,
                     const void *feats, const int32_t *cu_new, int32_t batch, int32_t rows,
                     void *ws, size_t ws_bytes, hipStream_t stream);

/* Drafting pass.  last_tok: [batch].  Block slot j of sequence s holds
 * last_tok[s] (j = 0) or dims->mask_id (j > 0) at rotary position
 * ctx_len[s] + j and attends to every cached position < ctx_len[s] and to
 * every block slot (ctx_len values above kv->capacity are read as
 * kv->capacity).  draft: [batch, B] out, the lowest-index argmax of the
 * shared lm_head logits per slot.  The cache is read, never written. */
int dflash_draft_forward(const dflash_dims *dims, const dflash_weights *w, const dflash_kv *kv,
                         const int32_t *last_tok, int32_t batch, int32_t *draft,
                         void *ws, size_t ws_bytes, hipStream_t stream);

/* Drafting passes over blocks with explicit anchors ("Term: DFlash
 * speculative decoding", "DFlash: architecture and workflow", stage one: the
 * engine picks anchor positions at the decoding frontier and at additional
 * points when several blocks are drafted concurrently).  Block a drafts for
 * cached sequence anchor_seq[a] in [0, kv->max_batch): slot 0 holds
 * anchor_tok[a] at rotary position p = anchor_pos[a], slot j > 0 holds
 * dims->mask_id at p + j, and the block attends to that sequence's cached
 * positions [0, p) and to its own slots.  0 <= p <= ctx_len[anchor_seq[a]]
 * (p = ctx_len is the frontier, the dflash_draft_forward case); several
 * blocks may share a sequence and do not see each other.  An anchor outside
 * the cache sets DFLASH_STATUS_ANCHOR and is clamped into it.  anchor_seq,
 * anchor_pos, anchor_tok: [nblocks] device arrays; 1 <= nblocks <= 64; the
 * workspace must hold dflash_workspace_bytes(dims, nblocks, .).  draft:
 * [nblocks, B] out.  The cache is read, never written. */
int dflash_draft_anchors(const dflash_dims *dims, const dflash_weights *w, const dflash_kv *kv,
                         const int32_t *anchor_seq, const int32_t *anchor_pos, const int32_t *anchor_tok,
                         int32_t nblocks, int32_t *draft, void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------- target pass */

/* The target's verify pass ("Term: DFlash speculative decoding", "DFlash:
 * architecture and workflow", stage three: the target computes its own
 * logits at every block position; "DFlash, Diffusion LLMs, dLLM, MTP and
 * Speculative Decoding: A Deep Research Report", "Key points": the drafter
 * is conditioned on hidden features from several target layers).  The
 * target is a decoder of the drafter's layer type (weights packed by the
 * same calls, dims with up to 128 layers) with causal attention: row i of
 * sequence s holds tokens[s][i] at rotary position ctx_len[s] + i and sees
 * the cached positions [0, ctx_len[s]) and rows 0 .. i.  The rows' K/V are
 * written to the cache at ctx_len[s] + i (DFLASH_STATUS_CAPACITY past the
 * capacity); ctx_len is not changed (dflash_kv_commit keeps the accepted
 * rows).  Outputs, storage dtype: out_hidden [batch, rows, H], the final
 * normalised hidden states (dflash_verify_accept's target_hidden), and
 * out_feats [batch, rows, n_feat * H], the residual stream after layer
 * feat_layers[k] ([host] array, distinct indices in [0, n_layers)) in
 * columns [k H, (k + 1) H) (dflash_inject_kv's feature rows).  tokens:
 * [batch, rows] device int32.  parents: NULL for the causal chain, or a
 * draft tree [batch, rows] (parents[s][0] = -1, 0 <= parents[s][i] < i):
 * row i is a tree node at rotary position ctx_len[s] + depth(i) that sees
 * the cached positions, its ancestors and itself (the ancestor-only mask of
 * "LLMs hit ludicrous speed: diffusion decoding and dMoE supercharge AI
 * inference, shattering old benchmarks", DDTree paragraph; a malformed
 * parent sets DFLASH_STATUS_TREE and is read as row i - 1); its K/V still go
 * to cache slot ctx_len[s] + i.  1 <= rows <= 32 (bf16) or 16 (fp32); weights:
 * embed, final_norm and the layers of `tw` (w_fc, fc_norm, lm_head unused).
 * The workspace must hold dflash_target_workspace_bytes(dims, batch, rows). */
size_t dflash_target_workspace_bytes(const dflash_dims *dims, int32_t max_batch, int32_t rows);
int dflash_target_forward(const dflash_dims *dims, const dflash_weights *tw, const dflash_kv *kv,
                          const int32_t *tokens, const int32_t *parents, int32_t batch, int32_t rows,
                          const int32_t *feat_layers, int32_t n_feat, void *out_hidden, void *out_feats, void *ws,
                          size_t ws_bytes, hipStream_t stream);

/* Draft trees (the DDTree paragraph above): the drafting pass of
 * dflash_draft_forward with its logits kept (draft_logits [batch * B,
 * vocab], caller-owned), then per sequence the tree of the `nodes` best
 * continuations of last_tok[s] over the topk most probable tokens of each
 * slot, a continuation t_1 .. t_k scoring sum_j log softmax(l_j)(t_j);
 * built best-first from a heap, ties to the smaller depth, then the smaller
 * rank.  Outputs tree_tok and tree_parent [batch, nodes + 1]: node 0 is the
 * anchor (parent -1), every parent precedes its children.  1 <= topk <= 8,
 * 1 <= nodes <= 31 and at most the number of continuations of length 1..B. */
int dflash_draft_tree(const dflash_dims *dims, const dflash_weights *w, const dflash_kv *kv,
                      const int32_t *last_tok, int32_t batch, int32_t topk, int32_t nodes, float *draft_logits,
                      int32_t *tree_tok, int32_t *tree_parent, void *ws, size_t ws_bytes, hipStream_t stream);

/* Greedy acceptance over draft trees: the shared lm_head's lowest-index
 * argmax at each of the n tree rows of target_hidden [batch, n, H] (the
 * target's tree pass) into target_argmax [batch, n]; then from the root
 * down, the child (lowest-numbered) whose token equals the argmax at the
 * current node, while there is one.  accept_len [batch] = depth reached,
 * bonus [batch] = argmax at the last accepted node, path [batch, n] = the
 * accepted nodes from the root (-1 after them).  1 <= n <= 32. */
int dflash_tree_accept(const dflash_dims *dims, const void *lm_head, const void *target_hidden,
                       const int32_t *tree_tok, const int32_t *tree_parent, int32_t batch, int32_t n,
                       int32_t *target_argmax, int32_t *accept_len, int32_t *bonus, int32_t *path, void *ws,
                       size_t ws_bytes, hipStream_t stream);

/* After a tree pass: the K/V rows of path node k (cache slot ctx_len[s] +
 * path[s][k]) move to ctx_len[s] + k for k <= accept_len[s], in every layer
 * and KV head, then ctx_len[s] += accept_len[s] + 1.  n as for the pass. */
int dflash_kv_commit_path(const dflash_dims *dims, const dflash_kv *kv, const int32_t *path,
                          const int32_t *accept_len, int32_t batch, int32_t n, hipStream_t stream);

/* After verification: ctx_len[s] += min(max(accept_len[s] + 1, 0),
 * max_commit), at most kv->capacity (the accepted drafts and the target's
 * next token stay in the cache; the rest of the pass's rows are dropped). */
int dflash_kv_commit(const dflash_dims *dims, const dflash_kv *kv, const int32_t *accept_len, int32_t batch,
                     int32_t max_commit, hipStream_t stream);

/* Temperature sampling ("Term: DFlash speculative decoding", "DFlash:
 * architecture and workflow": the speculator fills masked positions with
 * sampled tokens and the target applies an acceptance criterion; "DFlash,
 * Diffusion LLMs, dLLM, MTP and Speculative Decoding: A Deep Research
 * Report", "DFlash benchmark results": temperature 1).  The criterion is the
 * standard speculative-sampling rule: with q_j = softmax(l_j / T) the
 * drafter's and p_j = softmax(l'_j / T) the target's distribution at slot
 * j, drafted token d_j is accepted with probability min(1, p_j(d_j) /
 * q_j(d_j)) in slot order; at the first rejected slot the next token is
 * drawn from the normalised residual max(0, p_j - q_j), and after B
 * accepted slots from p_B.  Random numbers are inputs: uniforms in (0, 1),
 * turned into Gumbel noise g = -log(-log u); a categorical draw is the
 * lowest-index argmax of log(weight) + g over the vocabulary.
 *
 * dflash_draft_sample: the drafting pass of dflash_draft_forward, but each
 * slot's token is drawn from q_j: draft[m] = argmax_v l_m(v) / T + g_m(v)
 * with u_draft [batch * B, vocab] the uniforms of row m = s * B + j.  The
 * head's fp32 logits l (before the temperature) go to draft_logits
 * [batch * B, vocab] (caller-owned, read again by dflash_verify_sample).
 * temperature > 0 (DFLASH_ERR_SHAPE otherwise). */
int dflash_draft_sample(const dflash_dims *dims, const dflash_weights *w, const dflash_kv *kv,
                        const int32_t *last_tok, int32_t batch, float temperature, const float *u_draft,
                        int32_t *draft, float *draft_logits, void *ws, size_t ws_bytes, hipStream_t stream);

/* dflash_verify_sample: the speculative-sampling verification of a sampled
 * draft.  target_hidden [batch, B+1, H] and lm_head as for
 * dflash_verify_accept; draft [batch, B] and draft_logits [batch * B, vocab]
 * from dflash_draft_sample at the same temperature; u_accept [batch, B] the
 * acceptance uniforms (slot j is accepted when u <= p_j(d_j) / q_j(d_j));
 * u_resid [batch, vocab] the uniforms of the one draw per sequence (from the
 * residual of the first rejected slot, else from p_B).  target_logits
 * [batch * (B+1), vocab] is caller-owned scratch (it receives the target's
 * logits).  Outputs: accept_len [batch] in [0, B] and next_tok [batch], the
 * token the step emits after the accepted prefix.  Drafted ids outside
 * [0, vocab) are clamped.  The workspace needs
 * dflash_workspace_bytes(dims, batch, .). */
int dflash_verify_sample(const dflash_dims *dims, const void *lm_head, const void *target_hidden,
                         const int32_t *draft, const float *draft_logits, int32_t batch, float temperature,
                         const float *u_accept, const float *u_resid, float *target_logits,
                         int32_t *accept_len, int32_t *next_tok, void *ws, size_t ws_bytes,
                         hipStream_t stream);

/* Greedy verification.  target_hidden: [batch, B+1, H] row-major, storage
 * dtype: the target's final hidden states at its pass over
 * [x, d_0, ..., d_{B-1}].  lm_head: dflash_pack_lm_head output.  Outputs:
 * target_argmax [batch, B+1] (lowest index on ties), accept_len [batch] =
 * first j < B with draft[s][j] != target_argmax[s][j], else B, and
 * bonus [batch] = target_argmax[s][accept_len[s]]. */
int dflash_verify_accept(const dflash_dims *dims, const void *lm_head, const void *target_hidden,
                         const int32_t *draft, int32_t batch, int32_t *target_argmax,
                         int32_t *accept_len, int32_t *bonus, void *ws, size_t ws_bytes,
                         hipStream_t stream);

/* Greedy verification for callers that cannot allocate (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation):
 * the same computation and outputs as dflash_verify_accept, with no
 * workspace argument.  Its scratch (the argmax key slots and an arrival
 * counter, 1 MiB) is a static device array of the library, one per GPU,
 * looked up and zero-filled by the first call on each device (on `stream`,
 * with that device current) and held until the process ends; the call
 * itself allocates nothing.  batch must be in [1, 64] (DFLASH_ERR_SHAPE
 * otherwise).  Every call on one GPU shares that scratch: two calls that
 * overlap on one GPU (different streams, or different threads without
 * ordering) race.  Pointers and outputs as for dflash_verify_accept. */
int dflash_verify_accept_noalloc(const dflash_dims *dims, const void *lm_head, const void *target_hidden,
                                 const int32_t *draft, int32_t batch, int32_t *target_argmax,
                                 int32_t *accept_len, int32_t *bonus, hipStream_t stream);

/* ---------------------------------------------------------------- misc */
const char *dflash_status_str(int status);
const char *dflash_last_error(void);
int dflash_abi_version(void);
/* sha256 (hex) of the sources and build flags this library was built from,
 * or "unknown"; lets a caller detect a stale build. */
const char *dflash_build_id(void);

#ifdef __cplusplus
}
#endif
#endif /* DFLASH_H */
