// Kernel parameter blocks and host-side launchers shared by the kernel
// translation units and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/dflash.h"

namespace dflash {

// The first bytes of every workspace hold the argmax key slots: zeroed once
// at initialisation, cleared again by every reader.
constexpr int ARGMAX_SLOTS = 64;     // atomic-max slots per row
constexpr int MAX_KEY_ROWS = 1088;   // 64 sequences x 17 verify rows
constexpr size_t WS_COUNTER_BYTES = size_t(1) << 20;
static_assert(size_t(MAX_KEY_ROWS) * ARGMAX_SLOTS * 8 <= WS_COUNTER_BYTES, "key slots exceed the fixed area");
constexpr int MAX_SEGMENTS = 16;
// Sequences of one launch (the largest batch the library takes) and rotary
// pairs of a head (head_dim <= 128).
constexpr int MAX_SEQS = 64;
constexpr int MAX_ROPE_HALF = 64;
// Arrival counter of the last-arriver handshakes, at the end of the fixed area.
constexpr size_t WS_ARRIVE_OFFSET = WS_COUNTER_BYTES - 256;
// Split-K: partial tiles in a workspace region of SPLIT_PART_BYTES (tiled
// launches split only while their units' fp32 tiles fit it: 256 of 128 x 256,
// 1024 of 64 x 128), and one arrival count per item (zero between launches,
// at most MAX_SPLIT_ITEMS) just below the arrive counter.
constexpr int MAX_SPLIT_UNITS = 256;
constexpr size_t SPLIT_TILE_BYTES = size_t(128) * 256 * 4;
constexpr size_t SPLIT_PART_BYTES = MAX_SPLIT_UNITS * SPLIT_TILE_BYTES;
constexpr int MAX_SPLIT_ITEMS = 8192;
constexpr size_t WS_SPLIT_CNT_OFFSET = WS_ARRIVE_OFFSET - MAX_SPLIT_ITEMS * 4;
static_assert(size_t(MAX_KEY_ROWS) * ARGMAX_SLOTS * 8 <= WS_SPLIT_CNT_OFFSET, "key slots overlap the split counts");
// The argmax finish and the injection commit run inside the GEMM launch (by
// its last workgroup to finish) when the launch runs on the skinny kernel,
// which takes at most this many rows (17 for draft and verify heads, 32 for
// injections); tiled launches finish in argmax_finish_kernel.
constexpr int FUSED_FINISH_ROWS = 32;

enum Epilogue : int {
  EPI_STORE = 0,   // out_f32[m, n] = y
  EPI_RESID = 1,   // out_f32[m, n] = resid[m, n] + y
  EPI_SWIGLU = 2,  // packed act[m, j] = silu(gate) * up (tiles alternate gate / up)
  EPI_QKV = 3,     // RoPE on q and k of the block; q -> qbuf, k/v -> kblk/vblk
  EPI_KVINJ = 4,   // RoPE on injected k; k/v appended to the cache
  EPI_ARGMAX = 5,  // lowest-index argmax over the vocabulary (+ acceptance)
  EPI_LOGITS = 6,  // fp32 logits out_f32[m, n] for n < vocab (temperature sampling)
};

struct ArgmaxFinishParams {
  unsigned long long *keys;
  int rows_per_seq, block, verify;
  int *tok_out;
  const int *draft_in;
  int *accept_len, *bonus;
};

struct GemmParams {
  // A operand: packed weights, one pointer per segment of seg_ntiles 16-row tiles.
  const char *w_seg[MAX_SEGMENTS];
  int seg_ntiles;
  // B operand: activations, packed (x_ld == 0) or row-major with x_ld elements per row.
  // Packed activations may carry xs = 2 planes (hi, lo) x_plane bytes apart.
  const char *x;
  int x_ld;
  int xs;
  size_t x_plane;
  int M, m_tiles, m_blocks, MT;
  int N, n_tiles, n_blocks, NB;
  int k_tiles;
  int grid_cap;               // persistent workgroups: at most one per compute unit
  // EPI_STORE / EPI_RESID
  float *out_f32;
  const float *resid;
  int ld_out;
  // EPI_SWIGLU (output planes out_planes, out_plane bytes apart)
  char *out_packed;
  int out_kt, out_planes;
  size_t out_plane;
  // EPI_QKV / EPI_KVINJ
  int block, n_q, n_kv, head_dim;
  int rope_on;
  double rope_turns[64];      // theta^(-2i/d) / (2 pi), i < head_dim / 2
  const int *ctx_len;
  char *qbuf, *kblk, *vblk;
  size_t q_plane;
  int q_planes;               // planes of q written for the attention (1, or 2 = hi + lo)
  int q_tiles;                // 16-row tiles of q per (sequence, head): 1 for a draft block, 2 for up to 32 rows
  // EPI_QKV of a causal pass: the new rows' K/V also go to the cache
  // (kcache / vcache, layer layer0) at position ctx_len[s] + j.
  int qkv_to_cache;
  // Tree rows: row m's rotary position is ctx_len[s] + row_pos[m] (its
  // depth) instead of ctx_len[s] + j; null: j.
  const int *row_pos;
  char *kcache, *vcache;
  int layer0, capacity, max_batch;
  const int *cu_new;
  int batch;
  unsigned *status;
  // EPI_ARGMAX
  int vocab;
  unsigned long long *keys;   // [rows][ARGMAX_SLOTS]
  // RMSNorm split across two launches.  The producer (EPI_STORE / EPI_RESID)
  // also writes its output rows y as packed (y * nx_gain) planes (rows
  // [M, nx_rows) zeroed) and per row and 16-column tile the sum of y^2 to
  // ssq_out[m * ssq_ld + tile].  The consumer multiplies its output rows by
  // 1 / sqrt(mean(y^2) + eps): from the tile sums itself (rs_ssq, one row
  // block) or from per-row values (rs_direct) made by rstd_kernel.
  char *nx_packed;
  const char *nx_gain;
  int nx_kt, nx_planes, nx_rows;
  size_t nx_plane;
  float *ssq_out;
  int ssq_ld;
  // EPI_STORE / EPI_RESID: a copy of the output rows in the storage type,
  // aux_out[m * aux_ld + n] (the target's captured features).
  char *aux_out;
  int aux_ld;
  const float *rs_ssq;
  const float *rs_direct;
  int rs_tiles, rs_K;
  float rs_eps;
  // Last-arriver tail (arrive set): every workgroup completes its memory
  // operations and then increments *arrive; the one that sees grid - 1 runs
  // the argmax finish (EPI_ARGMAX, fin) or the ctx_len commit (EPI_KVINJ),
  // and resets *arrive to 0.
  unsigned *arrive;
  ArgmaxFinishParams fin;
  int *ctx_len_w;             // EPI_KVINJ commit target (the same array as ctx_len)
  // Tiled launches (gemm_tiled holds): 16-row tiles held by the
  // packed activation buffer (loads past it are clamped), and the output
  // tile's token fragments (4 to 12; set by the launcher, which also
  // sets m_blocks and n_blocks for the tile it picks).
  int tiled, x_mtiles, tile_m;
  // Split-K (tiled launches): partial tiles and per-item arrival counts in the
  // workspace (both null: no split); ksplit is set by the launcher.
  float *part_ws;
  unsigned *part_cnt;
  int ksplit;
};

// Whether a consumer can reduce the RMSNorm tile sums itself: one row block
// whose rows x tiles fit the 8192-float LDS stage.
inline bool gemm_inline_rs_ok(int m_blocks, int MT, int hidden) {
  return m_blocks == 1 && MT * 16 * (hidden / 16) <= 8192;
}

// Whether a launch keeps its activations resident in registers: one row
// block and a wavefront K chunk of at most 16 tiles with MT * planes <= 2, or
// of at most 48 tiles with a single row tile and plane.
// k_tiles: the k range one workgroup covers (a split part's, with split-K).
inline bool gemm_resident_ok(int m_blocks, int MT, int planes, int k_tiles) {
  const int per = (k_tiles + 7) / 8;
  return m_blocks == 1 && ((MT * planes <= 2 && per <= 16) || (MT * planes == 1 && per <= 48));
}


struct AttnParams {
  const char *qbuf, *kblk, *vblk;   // per-step block operands
  size_t q_plane;                   // bytes between the q hi and lo planes
  int xs;                           // 2: q and P carried as hi + lo bf16 planes
  const char *kcache, *vcache;      // this layer's cache (sequence-major regions)
  const int *ctx_len;               // per block: cached positions it attends to
  const int *region_of;             // per block: its sequence's cache region (null: the block's own)
  float *part;                      // [batch][n_q][splits] partial records
  int block, n_q, n_kv, head_dim, group, splits, capacity;
  int head_split;                   // workgroups sharing one KV head's query group
  int q_tiles;                      // 16-row query tiles per sequence (block rows up to 16 * q_tiles)
  int sort_seqs;                    // 1: workgroups take the sequences longest context first
  int causal;                       // block row i sees block positions <= i only
  const unsigned *row_mask;         // tree rows: block row i sees block positions j with bit j set
  float scale_log2;                 // log2(e) / sqrt(head_dim)
  // merge
  float *attn_out;                  // fp32 [batch*block, n_q*d]
  char *xo;                         // packed T [.., n_q*d] for the output projection
  int xo_kt;
  size_t xo_plane;
};

// Block embedding: gathers the token rows and prepares the first RMSNorm the
// way a GEMM producer does (fp32 rows, packed rows * gain, tile sums).
struct EmbedParams {
  const char *embed;       // T [V, H]
  const int *last_tok;     // [batch]
  const int *tokens;       // [batch * block]: every row's token (a target pass); null: last_tok + mask
  int block, mask_id, vocab;
  unsigned *status;
  float *gathered;         // fp32 [M, H]
  const char *gain;        // T [H]
  int M, rows_pad, H;
  char *xpacked;           // packed T [rows_pad, H] of gathered * gain
  int x_kt, planes;        // planes: 1, or 2 (hi, lo) x_plane bytes apart
  size_t x_plane;
  float *ssq;              // [M, H / 16] tile sums of squares
  // Anchored blocks (anchor_pos set): block s drafts for cached sequence
  // anchor_seq[s] from position anchor_pos[s]; the first row's thread 0
  // checks both against the cache (DFLASH_STATUS_ANCHOR when outside it,
  // then clamped) and writes them to blk_region / blk_ctx, which the QKV
  // epilogue and the attention read.
  const int *anchor_seq, *anchor_pos, *ctx_len;
  int max_batch, capacity;
  int *blk_ctx, *blk_region;
};

// Temperature sampling (sampling.hip).  Logit rows are fp32 [rows][ld];
// uniforms u lie in (0, 1).  Gumbel-max: a row's sample is the lowest-index
// argmax of logit * inv_t - log(-log u).
struct SampleParams {
  const float *logits;          // draft: the rows sampled
  int ld, vocab, chunks;        // chunks of the vocabulary per row (<= ARGMAX_SLOTS)
  float inv_t;                  // 1 / temperature
  const float *u;               // draft: [rows][vocab] uniforms
  unsigned long long *keys;     // argmax key slots, [rows][ARGMAX_SLOTS]
  // speculative verification (one sequence per grid row)
  const float *q_logits, *p_logits;   // draft rows [b * B][ld], target rows [b * (B + 1)][ld]
  const float *lse_q, *lse_p;         // their log-sum-exp of logit * inv_t
  const int *draft;                   // [b][B]
  int block;
  const float *u_accept;              // [b][B]
  const float *u_resid;               // [b][vocab]
  int *accept_len;                    // [b] out
};
hipError_t launch_gumbel_draft(const SampleParams &p, int rows, hipStream_t s);
// lse[r] = log sum_v exp(logits[r][v] * inv_t), through chunk partials part
// [rows][chunks] (scratch).
hipError_t launch_row_lse(const float *logits, int ld, int vocab, float inv_t, int rows, int chunks, float2 *part,
                          float *lse, hipStream_t s);
hipError_t launch_spec_sample(const SampleParams &p, int batch, hipStream_t s);

// Vocabulary chunks per row of the top-K (its first launch); the workspace
// holds TOPK_CHUNKS * K keys per row for the second.
constexpr int TOPK_CHUNKS = 32;

// Draft trees (tree.hip).
// Per row of logits, the K most probable entries as (log-probability,
// index), highest first (lowest index on ties): topk_val / topk_idx
// [rows][K]; lse[row] the row's log-sum-exp.
hipError_t launch_row_topk(const float *logits, int ld, int vocab, int rows, int K, const float *lse,
                           unsigned long long *chunk_keys, float *topk_val, int *topk_idx, hipStream_t s);
// Best-first trees, one per sequence: from the top-K of its B slots
// (rows s * B + j), N nodes after the anchor; tree_tok / tree_parent
// [batch][N + 1].
hipError_t launch_tree_build(const float *topk_val, const int *topk_idx, const int *anchor, int batch, int B,
                             int K, int N, int *tree_tok, int *tree_parent, hipStream_t s);
// Node depths and ancestor masks of trees of n rows (parents[s][0] = -1,
// each parent before its child; a malformed parent sets status bit
// DFLASH_STATUS_TREE and is read as the previous node).
hipError_t launch_tree_prep(const int *parent, int batch, int n, int *depth, unsigned *mask, unsigned *status,
                            hipStream_t s);
// Greedy walk down each tree along the target's argmax: accept_len, bonus,
// path [batch][n] (node ids, -1 past the end).
hipError_t launch_tree_walk(const int *tree_tok, const int *parent, const int *target_argmax, int batch, int n,
                            int *accept_len, int *bonus, int *path, hipStream_t s);
// Move each sequence's accepted path rows (ctx_len + path[k]) to
// ctx_len + k in every layer and KV head, then ctx_len += accept_len + 1.
hipError_t launch_commit_path(int dtype, char *kcache, char *vcache, int *ctx_len, const int *path,
                              const int *accept_len, int batch, int n, int n_layers, int max_batch, int n_kv,
                              int capacity, int head_dim, hipStream_t s);

// Greedy verification with its scratch (argmax key slots and the arrival
// counter, at least WS_COUNTER_BYTES, zero on entry) at wsb: the body of
// dflash_verify_accept after its workspace check.  Returns a dflash_status.
int verify_with_ws(const dflash_dims *d, const void *lm_head, const void *target_hidden, const int32_t *draft,
                   int32_t batch, int32_t *target_argmax, int32_t *accept_len, int32_t *bonus, char *wsb,
                   size_t ws_bytes, hipStream_t stream);
// Record an error for dflash_last_error() and return `code` (DFLASH_ERR_HIP
// with the HIP error string for set_hip_error).
int set_error(int code, const char *msg);
int set_hip_error(hipError_t e, const char *what);

// Launchers (return hipError_t of the launch).
hipError_t launch_gemm(int dtype, int epi, const GemmParams &p, hipStream_t s);
hipError_t launch_gemm_tiled(int dtype, int epi, const GemmParams &p, hipStream_t s);
hipError_t launch_argmax_finish(const ArgmaxFinishParams &p, int batch, hipStream_t s);
hipError_t launch_attention(int dtype, const AttnParams &p, int batch, hipStream_t s);
hipError_t launch_attn_merge(int dtype, const AttnParams &p, int batch, hipStream_t s);
hipError_t launch_embed(int dtype, const EmbedParams &p, hipStream_t s);
// rs[m] = 1 / sqrt(mean(x_m^2) + eps) from tile sums ssq[m * tiles + t].
hipError_t launch_rstd(const float *ssq, int tiles, int K, float eps, int M, float *rs, hipStream_t s);
hipError_t launch_pack_matrix(int dtype, const void *src, int rows, int cols, void *dst,
                              int dst_tile_offset, int dst_tile_stride, int rot_head_dim,
                              int rot_rows, bool pairs, hipStream_t s);
hipError_t launch_kv_convert(int dtype, bool to_packed, void *packed_k, void *packed_v,
                             void *plain_k, void *plain_v, long long regions, int capacity,
                             int head_dim, hipStream_t s);
hipError_t launch_zero(void *p, size_t bytes, hipStream_t s);
// out[m] = x[m] / sqrt(mean(x[m]^2) + eps) * gain, rows of H, in the storage type.
hipError_t launch_rownorm(int dtype, const float *x, int M, int H, const void *gain, float eps, void *out,
                          hipStream_t s);
// ctx_len[s] += min(max(accept_len[s] + 1, 0), max_commit), at most capacity.
hipError_t launch_kv_commit(int *ctx_len, const int *accept_len, int batch, int max_commit, int capacity,
                            hipStream_t s);

}  // namespace dflash
