// C ABI: validation, workspace layout, launch plans and the three step calls.
#include <string.h>

#include <algorithm>
#include <cmath>
#include <string>

#include "common.hpp"
#include "kernels.hpp"

using namespace dflash;

namespace {

thread_local std::string g_err;

int fail(int code, const std::string &msg) {
  g_err = msg;
  return code;
}

int hip_fail(hipError_t e, const char *what) {
  return fail(DFLASH_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t packed_bytes(int dtype, long long rows, long long cols) {
  const int kt = kt_of(dtype);
  return size_t((rows + 15) / 16) * size_t((cols + kt - 1) / kt) * 1024;
}

constexpr int MAX_BATCH = 64;
constexpr int MAX_TARGET_LAYERS = 128;

// Launches of more rows than these use the tiled kernel: from two row tiles
// on, the skinny kernel's activation stream per item (every row tile and
// plane through each workgroup) outweighs the tiled kernel's LDS traffic and
// split-K partial tiles.  The draft and verify layer GEMMs switch above 17
// rows (one sequence's 16 draft and 17 verify rows stay skinny).  The injection
// GEMMs stay skinny up to 32 rows: there the skinny kernel's summation order
// is the same for every row count, so an injection split over two such calls
// writes the same cache bits as one call.
constexpr int STEP_TILED_MIN_ROWS = 17;
constexpr int INJECT_TILED_MIN_ROWS = 32;
// The heads (one activation plane) stay skinny up to 32 rows when two row
// tiles of their activations fit the registers (k chunks of at most 16
// tiles: hidden <= 4096 in bf16); otherwise they switch with the layer GEMMs.
constexpr int HEAD_TILED_MIN_ROWS = 32;

struct GemmPlan {
  int M, N, K;
  int MT, NB, m_tiles, m_blocks, n_tiles, n_blocks, k_tiles;
  bool tiled;
};

// nb: weight tiles per workgroup (2 for the gate/up pairs and the argmax,
// 1 otherwise); the workgroup's wavefronts split K.  Launches of more than
// tiled_above rows take the tiled kernel.
GemmPlan plan_gemm(int dtype, int M, int N, int K, int nb, int tiled_above) {
  GemmPlan g{};
  g.tiled = M > tiled_above;
  g.M = M;
  g.N = N;
  g.K = K;
  const int kt = kt_of(dtype);
  g.m_tiles = (M + 15) / 16;
  g.MT = g.m_tiles <= 1 ? 1 : (g.m_tiles <= 2 ? 2 : 4);
  g.m_blocks = std::max(1, (g.m_tiles + g.MT - 1) / g.MT);
  g.NB = nb;
  g.n_tiles = (N + 15) / 16;
  g.n_blocks = (g.n_tiles + g.NB - 1) / g.NB;
  g.k_tiles = (K + kt - 1) / kt;
  return g;
}

int compute_units();

// Draft, verify and target layer GEMMs: skinny up to 17 rows; at 18-32 rows
// (two row tiles) skinny when its items fill at least half of their last
// round on the compute units (one item per workgroup at a time; a short last
// round leaves the skinny kernel's two-row-tile items, which stream their
// activations, less balanced than the tiled kernel's split-K parts), else
// tiled.
GemmPlan plan_layer(int dtype, int M, int N, int K, int nb) {
  GemmPlan g = plan_gemm(dtype, M, N, K, nb, STEP_TILED_MIN_ROWS);
  if (g.tiled && M <= 32) {
    const int cu = compute_units();
    const int rem = g.n_blocks % cu;
    if (rem == 0 || 2 * rem >= cu) g.tiled = false;
  }
  return g;
}

GemmPlan plan_head(int dtype, int M, int vocab, int hidden) {
  const int k_tiles = (hidden + kt_of(dtype) - 1) / kt_of(dtype);
  const bool resident = gemm_resident_ok(1, 2, 1, k_tiles);
  return plan_gemm(dtype, M, vocab, hidden, 2, resident ? HEAD_TILED_MIN_ROWS : STEP_TILED_MIN_ROWS);
}

// Context splits of the block attention: about half a workgroup per compute
// unit over all (sequence, KV head) pairs, at most 16 (more splits cost the
// merge more than they save here).  Pairs that fill the compute units on
// their own are split in two, so that with the longest contexts dispatched
// first (sort_seqs) the halves of a ragged batch pack the compute units
// instead of its longest sequence setting the launch's length.
int attn_splits(const dflash_dims *d, int batch) {
  const int s = 256 / std::max(1, batch * d->n_kv_heads);
  if (s <= 1 && batch > 1) return 2;
  return std::min(16, std::max(1, s));
}

// Workgroups per (sequence, KV head, split) sharing the query group: the
// largest divisor of the group that keeps the grid within 256 workgroups.
int attn_head_split(const dflash_dims *d, int batch, int splits) {
  const int group = d->n_q_heads / d->n_kv_heads;
  const int wgs = batch * d->n_kv_heads * splits;
  int best = 1;
  for (int hs = 1; hs <= group; ++hs)
    if (group % hs == 0 && wgs * hs <= 256) best = hs;
  return best;
}

struct Bump {
  size_t off = WS_COUNTER_BYTES;
  size_t take(size_t bytes) {
    off = (off + 255) & ~size_t(255);
    const size_t r = off;
    off += bytes;
    return r;
  }
};

// bf16 activations produced inside the step travel as hi + lo planes (about
// 16 mantissa bits).  The SwiGLU output feeds only the down projection: one
// bf16 plane there adds about 0.1% to each layer's residual, which over 8
// layers moves logits by close to the 1e-2 gap at which drafted tokens are
// decided, so launches of more than one 16-row tile carry two planes; a
// single row tile (one sequence of a 16-slot block) carries one, which lets
// the down projection keep its whole activation chunk in registers (a second
// plane would double the activation bytes every workgroup streams there).
// At 64 rows over 16384 cached positions a single plane left a drafted token
// with a 0.0108 logit gap on the wrong side.
constexpr int MLP_ONE_PLANE_ROWS = 16;
int act_planes(const dflash_dims *d) { return d->dtype == DFLASH_BF16 ? 2 : 1; }
int mlp_act_planes(const dflash_dims *d, int rows) { return rows > MLP_ONE_PLANE_ROWS ? act_planes(d) : 1; }

struct DraftLayout {
  size_t hidden, mid, attn, xa, xo, xact, qbuf, kblk, vblk, apart, ssq, rs, part, anc, tree, end;
  size_t pa, po, pact, pq;  // bytes of one plane of xa, xo, xact, qbuf
  int M, Mp, S, xs, act_xs;  // planes of the packed activations and of the SwiGLU output
  int rows, q_tiles;         // rows per sequence; 16-row query tiles per sequence
  bool rs_inline;  // consumers reduce the RMSNorm tile sums themselves (one row block)
  GemmPlan qkv, o, gu, down, lm;
};

// Workspace of a layer stack over `batch` sequences of `rows` rows: the
// drafting pass (rows = B; every layer's residuals and attention output are
// kept for the views) or the target's causal pass (target: rows up to 32,
// two residual buffers used in turn and one attention output).
DraftLayout draft_layout(const dflash_dims *d, int batch, int rows = 0, bool target = false) {
  DraftLayout L{};
  const int es = esize_of(d->dtype), kt = kt_of(d->dtype);
  const int H = d->hidden, NQD = d->n_q_heads * d->head_dim, I = d->intermediate, hd = d->head_dim;
  L.rows = rows > 0 ? rows : d->block_size;
  L.q_tiles = (L.rows + 15) / 16;
  L.M = batch * L.rows;
  L.S = attn_splits(d, batch * L.q_tiles);
  L.qkv = plan_layer(d->dtype, L.M, (d->n_q_heads + 2 * d->n_kv_heads) * hd, H, 1);
  L.o = plan_layer(d->dtype, L.M, H, NQD, 1);
  L.gu = plan_layer(d->dtype, L.M, 2 * I, H, 2);
  L.down = plan_layer(d->dtype, L.M, H, I, 1);
  L.lm = plan_head(d->dtype, L.M, d->vocab, H);
  // packed activations hold whole row blocks (the GEMMs load them unguarded)
  L.Mp = L.qkv.m_blocks * L.qkv.MT * 16;
  Bump b;
  const size_t row = size_t(L.M) * H * 4;
  L.hidden = b.take(row * (target ? 2 : d->n_layers + 1));
  L.mid = b.take(row * (target ? 1 : d->n_layers));
  L.attn = b.take(size_t(L.M) * NQD * 4 * (target ? 1 : d->n_layers));
  L.ssq = b.take(size_t(L.M) * (H / 16) * 4);
  L.rs = b.take(size_t(L.M) * 4);
  L.xs = act_planes(d);
  L.pa = packed_bytes(d->dtype, L.Mp, H);
  L.po = packed_bytes(d->dtype, L.Mp, NQD);
  L.pact = packed_bytes(d->dtype, L.Mp, I);
  L.pq = size_t(batch) * d->n_q_heads * L.q_tiles * (hd / kt) * 1024;
  L.xa = b.take(L.pa * L.xs);
  L.xo = b.take(L.po * L.xs);
  L.act_xs = mlp_act_planes(d, L.M);
  L.xact = b.take(L.pact * L.act_xs);
  L.qbuf = b.take(L.pq * L.xs);
  L.kblk = b.take(size_t(batch) * d->n_kv_heads * kt * hd * es);
  L.vblk = b.take(size_t(batch) * d->n_kv_heads * kt * hd * es);
  L.apart = b.take(size_t(batch) * L.q_tiles * d->n_q_heads * L.S * ((hd / 16) * 1024 + 128));
  L.rs_inline = gemm_inline_rs_ok(L.qkv.m_blocks, L.qkv.MT, H);
  L.part = L.M > STEP_TILED_MIN_ROWS ? b.take(SPLIT_PART_BYTES) : 0;
  L.anc = b.take(size_t(2) * MAX_BATCH * 4);   // anchored blocks: checked context lengths, cache regions
  // draft trees: per slot row the log-sum-exp, its chunk partials, the
  // top-K (value, index) and the top-K chunk keys; target tree passes: per
  // row depth and ancestor mask
  L.tree = b.take(size_t(L.M) * (4 + ARGMAX_SLOTS * 8 + 8 * 8 + TOPK_CHUNKS * 8 * 8) + size_t(L.M) * 8);
  L.end = b.off;
  return L;
}

struct VerifyLayout {
  size_t lse, lse_part, end;
  GemmPlan lm;
};

// The greedy verify call needs the counter area only; the sampling one adds
// the log-sum-exp of its batch * (2B + 1) logit rows.
VerifyLayout verify_layout(const dflash_dims *d, int batch, bool sampling = false) {
  VerifyLayout L{};
  L.lm = plan_head(d->dtype, batch * (d->block_size + 1), d->vocab, d->hidden);
  Bump b;
  L.lse = sampling ? b.take(size_t(batch) * (2 * d->block_size + 1) * 4) : 0;
  // chunk partials of the log-sum-exp (one float2 per row and chunk)
  L.lse_part = sampling ? b.take(size_t(batch) * (2 * d->block_size + 1) * ARGMAX_SLOTS * 8) : 0;
  L.end = sampling ? b.off : WS_COUNTER_BYTES;
  return L;
}

// Vocabulary chunks per row of the sampling kernels: about 2048 entries
// each, at most one per argmax slot.
int sample_chunks(int vocab) { return std::max(1, std::min(ARGMAX_SLOTS, (vocab + 2047) / 2048)); }

struct InjectLayout {
  size_t u, xc, ssq, rs, part, end, pc;
  int Rp, xs;
  bool rs_inline;
  GemmPlan fc, kv;
};

InjectLayout inject_layout(const dflash_dims *d, int rows) {
  InjectLayout L{};
  const int H = d->hidden;

  L.fc = plan_gemm(d->dtype, rows, H, d->n_feat_layers * H, 1, INJECT_TILED_MIN_ROWS);
  L.kv = plan_gemm(d->dtype, rows, d->n_layers * 2 * d->n_kv_heads * d->head_dim, H, 1, INJECT_TILED_MIN_ROWS);
  L.Rp = L.kv.m_blocks * L.kv.MT * 16;
  Bump b;
  L.u = b.take(size_t(rows) * H * 4);
  L.ssq = b.take(size_t(rows) * (H / 16) * 4);
  L.rs = b.take(size_t(rows) * 4);
  L.xs = act_planes(d);
  L.pc = packed_bytes(d->dtype, L.Rp, H);
  L.xc = b.take(L.pc * L.xs);
  L.rs_inline = gemm_inline_rs_ok(L.kv.m_blocks, L.kv.MT, H);
  L.part = rows > INJECT_TILED_MIN_ROWS ? b.take(SPLIT_PART_BYTES) : 0;
  L.end = b.off;
  return L;
}

int check_dims(const dflash_dims *d, int max_layers = MAX_SEGMENTS) {
  if (!d) return fail(DFLASH_ERR_NULL, "dims is NULL");
  if (d->dtype != DFLASH_BF16 && d->dtype != DFLASH_F32) return fail(DFLASH_ERR_DTYPE, "dtype must be DFLASH_BF16 or DFLASH_F32");
  // Malformed dimensions: DFLASH_ERR_SHAPE.
  if (d->hidden <= 0 || d->hidden % 32) return fail(DFLASH_ERR_SHAPE, "hidden must be a positive multiple of 32");
  if (d->head_dim <= 0 || d->head_dim % 32) return fail(DFLASH_ERR_SHAPE, "head_dim must be a positive multiple of 32");
  if (d->n_kv_heads <= 0 || d->n_q_heads <= 0 || d->n_q_heads % d->n_kv_heads) return fail(DFLASH_ERR_SHAPE, "n_q_heads must be a positive multiple of n_kv_heads");
  if (d->n_layers < 1) return fail(DFLASH_ERR_SHAPE, "n_layers must be >= 1");
  if (d->intermediate <= 0 || d->intermediate % 32) return fail(DFLASH_ERR_SHAPE, "intermediate must be a positive multiple of 32");
  if (d->n_feat_layers < 1) return fail(DFLASH_ERR_SHAPE, "n_feat_layers must be >= 1");
  if (d->vocab < 32 || d->vocab % 32) return fail(DFLASH_ERR_SHAPE, "vocab must be a positive multiple of 32");
  if (d->mask_id < 0 || d->mask_id >= d->vocab) return fail(DFLASH_ERR_SHAPE, "mask_id must be in [0, vocab)");
  if (d->block_size < 1 || d->block_size > 16) return fail(DFLASH_ERR_SHAPE, "block_size must be in [1, 16]");
  if (!(d->rms_eps >= 0.f) || !(d->rope_theta >= 0.f)) return fail(DFLASH_ERR_SHAPE, "rms_eps and rope_theta must be >= 0");
  // Well-formed but outside what the kernels are built for: DFLASH_ERR_UNSUPPORTED.
  if (d->hidden % 64 || d->hidden > 8192) return fail(DFLASH_ERR_UNSUPPORTED, "hidden must be a multiple of 64, at most 8192");
  if (d->head_dim != 64 && d->head_dim != 128) return fail(DFLASH_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (d->n_q_heads / d->n_kv_heads > 16) return fail(DFLASH_ERR_UNSUPPORTED, "at most 16 query heads per KV head");
  if (d->n_layers > max_layers)
    return fail(DFLASH_ERR_UNSUPPORTED, max_layers == MAX_SEGMENTS ? "at most 16 layers" : "at most 128 target layers");
  return DFLASH_OK;
}

int check_kv(const dflash_dims *d, const dflash_kv *kv) {
  if (!kv) return fail(DFLASH_ERR_NULL, "kv is NULL");
  if (!kv->k || !kv->v || !kv->ctx_len || !kv->status) return fail(DFLASH_ERR_NULL, "kv->k, v, ctx_len and status must be set");
  if (!aligned16(kv->k) || !aligned16(kv->v)) return fail(DFLASH_ERR_ALIGN, "kv->k and kv->v must be 16-byte aligned");
  if (kv->capacity <= 0 || kv->capacity % 32) return fail(DFLASH_ERR_SHAPE, "kv->capacity must be a positive multiple of 32");
  if (kv->max_batch < 1 || kv->max_batch > MAX_BATCH) return fail(DFLASH_ERR_SHAPE, "kv->max_batch must be in [1, 64]");
  (void)d;
  return DFLASH_OK;
}

int check_ptr(const void *p, const char *name, bool align = true) {
  if (!p) return fail(DFLASH_ERR_NULL, std::string(name) + " is NULL");
  if (align && !aligned16(p)) return fail(DFLASH_ERR_ALIGN, std::string(name) + " must be 16-byte aligned");
  return DFLASH_OK;
}

#define TRY(x)                 \
  do {                         \
    const int _r = (x);        \
    if (_r != DFLASH_OK) return _r; \
  } while (0)

int check_weights(const dflash_dims *d, const dflash_weights *w, bool need_fc, bool need_draft) {
  if (!w) return fail(DFLASH_ERR_NULL, "weights is NULL");
  if (!w->layers) return fail(DFLASH_ERR_NULL, "weights->layers is NULL");
  if (need_fc) {
    TRY(check_ptr(w->w_fc, "w_fc"));
    TRY(check_ptr(w->fc_norm, "fc_norm"));
  }
  if (need_draft) {
    TRY(check_ptr(w->embed, "embed"));
    TRY(check_ptr(w->final_norm, "final_norm"));
    TRY(check_ptr(w->lm_head, "lm_head"));
  }
  for (int l = 0; l < d->n_layers; ++l) {
    const dflash_layer &L = w->layers[l];
    TRY(check_ptr(L.w_qkv, "layers[].w_qkv"));
    if (need_draft) {
      TRY(check_ptr(L.attn_norm, "layers[].attn_norm"));
      TRY(check_ptr(L.w_o, "layers[].w_o"));
      TRY(check_ptr(L.mlp_norm, "layers[].mlp_norm"));
      TRY(check_ptr(L.w_gate_up, "layers[].w_gate_up"));
      TRY(check_ptr(L.w_down, "layers[].w_down"));
    }
  }
  return DFLASH_OK;
}

// Compute units of the current device (cached per device): the persistent
// GEMM launches at most one workgroup per compute unit.
int compute_units() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// Rotary frequencies in turns per position, in fp64: theta^(-2i/d) / (2 pi).
void fill_rope(GemmParams &p, const dflash_dims *d) {
  p.rope_on = d->rope_theta != 0.f;
  const int half = d->head_dim / 2;
  for (int i = 0; i < half && i < 64; ++i)
    p.rope_turns[i] = std::pow(double(d->rope_theta), -2.0 * i / d->head_dim) / (2.0 * M_PI);
}

// Producer half of an RMSNorm: the launch's fp32 output rows also go out as
// packed (rows * gain) planes of rows_pad rows and as tile sums of squares.
void set_norm_out(GemmParams &p, char *packed, int kt_count, int planes, size_t plane_bytes, int rows_pad,
                  const void *gain, float *ssq) {
  p.nx_packed = packed;
  p.nx_kt = kt_count;
  p.nx_planes = planes;
  p.nx_plane = plane_bytes;
  p.nx_rows = rows_pad;
  p.nx_gain = static_cast<const char *>(gain);
  p.ssq_out = ssq;
  p.ssq_ld = p.N / 16;
}

// Consumer half: scale the output rows by 1 / rms from the producer's tile
// sums, inline for one row block, else through rstd_kernel (one launch).
hipError_t set_norm_in(GemmParams &p, bool inline_rs, const float *ssq, float *rs, int M, int H, float eps,
                       hipStream_t stream) {
  p.rs_tiles = H / 16;
  p.rs_K = H;
  p.rs_eps = eps;
  if (inline_rs && !p.tiled) {   // the tiled kernel reads per-row scales only
    p.rs_ssq = ssq;
    return hipSuccess;
  }
  p.rs_direct = rs;
  return launch_rstd(ssq, H / 16, H, eps, M, rs, stream);
}

// The head GEMM with its argmax finish: inside the launch (last arriver of
// the skinny kernel) for at most FUSED_FINISH_ROWS rows, else as a follow-up
// kernel per sequence.
int launch_argmax_head(int dtype, GemmParams &lm, const ArgmaxFinishParams &fp, char *wsb, int batch,
                       hipStream_t stream, const char *what) {
  const bool fused = !lm.tiled && lm.M <= FUSED_FINISH_ROWS;
  if (fused) {
    lm.arrive = reinterpret_cast<unsigned *>(wsb + WS_ARRIVE_OFFSET);
    lm.fin = fp;
  }
  hipError_t e = launch_gemm(dtype, EPI_ARGMAX, lm, stream);
  if (e == hipSuccess && !fused) e = launch_argmax_finish(fp, batch, stream);
  if (e != hipSuccess) return hip_fail(e, what);
  return DFLASH_OK;
}

// Split-K scratch of a many-row launch: partial tiles at ws + part (0: the
// layout has none) and the per-item counts in the fixed counter area.
void set_split(GemmParams &p, char *wsb, size_t part) {
  p.part_ws = part ? reinterpret_cast<float *>(wsb + part) : nullptr;
  p.part_cnt = part ? reinterpret_cast<unsigned *>(wsb + WS_SPLIT_CNT_OFFSET) : nullptr;
}

void fill_gemm(GemmParams &p, const GemmPlan &g) {
  p.grid_cap = compute_units();
  p.M = g.M;
  p.N = g.N;
  p.m_tiles = g.m_tiles;
  p.m_blocks = g.m_blocks;
  p.MT = g.MT;
  p.n_tiles = g.n_tiles;
  p.n_blocks = g.n_blocks;
  p.NB = g.NB;
  p.k_tiles = g.k_tiles;
  p.seg_ntiles = g.n_tiles;
  p.xs = 1;
  p.out_planes = 1;
  // packed activation buffers hold whole row blocks of the row-tile plan
  p.x_mtiles = g.m_blocks * g.MT;
  // the tiled kernel picks its tile shape
  if (g.tiled) p.tiled = 1;
}

// One decoder layer of the drafting pass or of the target's causal pass:
// QKV with RoPE, the attention (and its split merge), o_proj with the
// residual, gate/up with SwiGLU and down with the residual.  RMSNorms are
// split between producer and consumer launches; the down projection produces
// the next layer's input norm (next_gain).
struct LayerRun {
  const dflash_dims *d;
  const DraftLayout *L;
  char *wsb;
  int batch;
  const int *ctx_of;            // per sequence: cached positions attended (rotary base)
  const int *region_of;         // per sequence: its cache region (null: its own)
  const char *kcache, *vcache;  // the whole cache; layer l at l * region_layer
  size_t region_layer;
  int capacity, max_batch;
  bool causal;                  // target pass: causal block, new K/V appended to the cache
  const int *row_pos;           // tree pass: per-row depth (rotary offset)
  const unsigned *row_mask;     // tree pass: per-row ancestor mask
  unsigned *status;
  const char *what;
};

int run_layer(const LayerRun &r, const dflash_layer &lw, int l, const void *next_gain, float *h_in, float *h_mid,
              float *h_out, float *attn_out, char *aux_out, int aux_ld, hipStream_t stream) {
  const dflash_dims *d = r.d;
  const DraftLayout &L = *r.L;
  char *wsb = r.wsb;
  const int H = d->hidden, kt = kt_of(d->dtype), hd = d->head_dim;
  const int NQD = d->n_q_heads * hd, I = d->intermediate;
  float *ssq = reinterpret_cast<float *>(wsb + L.ssq);
  float *rs = reinterpret_cast<float *>(wsb + L.rs);
  const std::string what(r.what);
  hipError_t e;

  GemmParams q{};
  fill_gemm(q, L.qkv);
  set_split(q, wsb, L.part);
  q.w_seg[0] = static_cast<const char *>(lw.w_qkv);
  q.x = wsb + L.xa;
  q.xs = L.xs;
  q.x_plane = L.pa;
  q.q_plane = L.pq;
  q.q_planes = L.xs;   // q itself goes to the attention as hi + lo
  q.q_tiles = L.q_tiles;
  q.block = L.rows;
  q.n_q = d->n_q_heads;
  q.n_kv = d->n_kv_heads;
  q.head_dim = hd;
  fill_rope(q, d);
  q.ctx_len = r.ctx_of;
  q.qbuf = wsb + L.qbuf;
  q.kblk = wsb + L.kblk;
  q.vblk = wsb + L.vblk;
  if (r.causal) {
    q.qkv_to_cache = 1;
    q.kcache = const_cast<char *>(r.kcache);
    q.vcache = const_cast<char *>(r.vcache);
    q.layer0 = l;
    q.capacity = r.capacity;
    q.max_batch = r.max_batch;
    q.status = r.status;
    q.row_pos = r.row_pos;
  }
  e = set_norm_in(q, L.rs_inline, ssq, rs, L.M, H, d->rms_eps, stream);
  if (e == hipSuccess) e = launch_gemm(d->dtype, EPI_QKV, q, stream);
  if (e != hipSuccess) return hip_fail(e, (what + " qkv").c_str());

  AttnParams a{};
  a.qbuf = wsb + L.qbuf;
  a.q_plane = L.pq;
  a.xs = L.xs;
  a.xo_plane = L.po;
  a.kblk = wsb + L.kblk;
  a.vblk = wsb + L.vblk;
  a.kcache = r.kcache + r.region_layer * l;
  a.vcache = r.vcache + r.region_layer * l;
  a.ctx_len = r.ctx_of;
  a.region_of = r.region_of;
  a.part = reinterpret_cast<float *>(wsb + L.apart);
  a.block = L.rows;
  a.q_tiles = L.q_tiles;
  a.causal = r.causal && !r.row_mask ? 1 : 0;
  a.row_mask = r.row_mask;
  a.n_q = d->n_q_heads;
  a.n_kv = d->n_kv_heads;
  a.head_dim = hd;
  a.group = d->n_q_heads / d->n_kv_heads;
  a.splits = L.S;
  a.head_split = attn_head_split(d, r.batch * L.q_tiles, L.S);
  // more workgroups than compute units: the longest contexts go first
  a.sort_seqs = r.batch > 1 && L.S * r.batch * L.q_tiles * d->n_kv_heads * a.head_split > compute_units() ? 1 : 0;
  a.capacity = r.capacity;
  a.scale_log2 = 1.4426950408889634f / sqrtf(float(hd));
  a.attn_out = attn_out;
  a.xo = wsb + L.xo;
  a.xo_kt = NQD / kt;
  e = launch_attention(d->dtype, a, r.batch, stream);
  if (e != hipSuccess) return hip_fail(e, (what + " attention").c_str());
  if (a.splits > 1) {
    e = launch_attn_merge(d->dtype, a, r.batch, stream);
    if (e != hipSuccess) return hip_fail(e, (what + " attention merge").c_str());
  }

  GemmParams o{};
  fill_gemm(o, L.o);
  set_split(o, wsb, L.part);
  o.w_seg[0] = static_cast<const char *>(lw.w_o);
  o.x = wsb + L.xo;
  o.xs = L.xs;
  o.x_plane = L.po;
  o.out_f32 = h_mid;
  o.resid = h_in;
  o.ld_out = H;
  set_norm_out(o, wsb + L.xa, H / kt, L.xs, L.pa, L.Mp, lw.mlp_norm, ssq);
  e = launch_gemm(d->dtype, EPI_RESID, o, stream);
  if (e != hipSuccess) return hip_fail(e, (what + " o_proj").c_str());

  GemmParams gu{};
  fill_gemm(gu, L.gu);
  set_split(gu, wsb, L.part);
  gu.w_seg[0] = static_cast<const char *>(lw.w_gate_up);
  gu.x = wsb + L.xa;
  gu.xs = L.xs;
  gu.x_plane = L.pa;
  gu.out_planes = L.act_xs;
  gu.out_plane = L.pact;
  gu.out_packed = wsb + L.xact;
  gu.out_kt = I / kt;
  e = set_norm_in(gu, L.rs_inline, ssq, rs, L.M, H, d->rms_eps, stream);
  if (e == hipSuccess) e = launch_gemm(d->dtype, EPI_SWIGLU, gu, stream);
  if (e != hipSuccess) return hip_fail(e, (what + " gate_up").c_str());

  GemmParams dn{};
  fill_gemm(dn, L.down);
  set_split(dn, wsb, L.part);
  dn.w_seg[0] = static_cast<const char *>(lw.w_down);
  dn.x = wsb + L.xact;
  dn.xs = L.act_xs;
  dn.x_plane = L.pact;
  dn.out_f32 = h_out;
  dn.resid = h_mid;
  dn.ld_out = H;
  dn.aux_out = aux_out;
  dn.aux_ld = aux_ld;
  set_norm_out(dn, wsb + L.xa, H / kt, L.xs, L.pa, L.Mp, next_gain, ssq);
  e = launch_gemm(d->dtype, EPI_RESID, dn, stream);
  if (e != hipSuccess) return hip_fail(e, (what + " down").c_str());
  return DFLASH_OK;
}

}  // namespace

namespace dflash {

int set_error(int code, const char *msg) { return fail(code, msg); }

int set_hip_error(hipError_t e, const char *what) { return hip_fail(e, what); }

int verify_with_ws(const dflash_dims *d, const void *lm_head, const void *target_hidden, const int32_t *draft,
                int32_t batch, int32_t *target_argmax, int32_t *accept_len, int32_t *bonus, char *wsb,
                size_t ws_bytes, hipStream_t stream) {
  TRY(check_dims(d));
  TRY(check_ptr(lm_head, "lm_head"));
  TRY(check_ptr(target_hidden, "target_hidden"));
  TRY(check_ptr(draft, "draft", false));
  TRY(check_ptr(target_argmax, "target_argmax", false));
  TRY(check_ptr(accept_len, "accept_len", false));
  TRY(check_ptr(bonus, "bonus", false));
  if (batch < 1 || batch > MAX_BATCH) return fail(DFLASH_ERR_SHAPE, "batch must be in [1, 64]");
  const VerifyLayout L = verify_layout(d, batch);
  if (ws_bytes < L.end) return fail(DFLASH_ERR_WORKSPACE, "workspace too small for this batch");
  GemmParams lm{};
  fill_gemm(lm, L.lm);
  lm.w_seg[0] = static_cast<const char *>(lm_head);
  lm.x = static_cast<const char *>(target_hidden);
  lm.x_ld = d->hidden;
  lm.vocab = d->vocab;
  lm.keys = reinterpret_cast<unsigned long long *>(wsb);
  ArgmaxFinishParams fp{};
  fp.keys = lm.keys;
  fp.rows_per_seq = d->block_size + 1;
  fp.block = d->block_size;
  fp.verify = 1;
  fp.tok_out = target_argmax;
  fp.draft_in = draft;
  fp.accept_len = accept_len;
  fp.bonus = bonus;
  return launch_argmax_head(d->dtype, lm, fp, wsb, batch, stream, "verify");
}

}  // namespace dflash

extern "C" {

int dflash_abi_version(void) { return DFLASH_ABI_VERSION; }

#ifndef DFLASH_SOURCE_DIGEST
#define DFLASH_SOURCE_DIGEST "unknown"
#endif
const char *dflash_build_id(void) { return DFLASH_SOURCE_DIGEST; }

const char *dflash_last_error(void) { return g_err.c_str(); }

const char *dflash_status_str(int s) {
  switch (s) {
    case DFLASH_OK: return "ok";
    case DFLASH_ERR_NULL: return "null pointer";
    case DFLASH_ERR_SHAPE: return "bad shape";
    case DFLASH_ERR_DTYPE: return "bad dtype";
    case DFLASH_ERR_WORKSPACE: return "workspace too small";
    case DFLASH_ERR_ALIGN: return "misaligned pointer";
    case DFLASH_ERR_HIP: return "HIP error";
    case DFLASH_ERR_UNSUPPORTED: return "unsupported";
    default: return "unknown status";
  }
}

size_t dflash_packed_bytes(int32_t dtype, int32_t rows, int32_t cols) {
  if ((dtype != DFLASH_BF16 && dtype != DFLASH_F32) || rows <= 0 || cols <= 0) return 0;
  return packed_bytes(dtype, rows, cols);
}

int dflash_pack_matrix(int32_t dtype, const void *src, int32_t rows, int32_t cols, void *dst, hipStream_t stream) {
  if (dtype != DFLASH_BF16 && dtype != DFLASH_F32) return fail(DFLASH_ERR_DTYPE, "bad dtype");
  if (rows <= 0 || cols <= 0) return fail(DFLASH_ERR_SHAPE, "rows and cols must be positive");
  TRY(check_ptr(src, "src"));
  TRY(check_ptr(dst, "dst"));
  if ((size_t(cols) * esize_of(dtype)) % 16) return fail(DFLASH_ERR_ALIGN, "row pitch must be a multiple of 16 bytes");
  const hipError_t e = launch_pack_matrix(dtype, src, rows, cols, dst, 0, 1, 1, 0, false, stream);
  return e == hipSuccess ? DFLASH_OK : hip_fail(e, "pack_matrix");
}

int dflash_pack_lm_head(int32_t dtype, const void *src, int32_t vocab, int32_t hidden, void *dst, hipStream_t stream) {
  if (dtype != DFLASH_BF16 && dtype != DFLASH_F32) return fail(DFLASH_ERR_DTYPE, "bad dtype");
  if (vocab <= 0 || vocab % 32 || hidden <= 0) return fail(DFLASH_ERR_SHAPE, "vocab must be a positive multiple of 32");
  TRY(check_ptr(src, "src"));
  TRY(check_ptr(dst, "dst"));
  if ((size_t(hidden) * esize_of(dtype)) % 16) return fail(DFLASH_ERR_ALIGN, "row pitch must be a multiple of 16 bytes");
  const hipError_t e = launch_pack_matrix(dtype, src, vocab, hidden, dst, 0, 1, 1, 0, true, stream);
  return e == hipSuccess ? DFLASH_OK : hip_fail(e, "pack_lm_head");
}

int dflash_pack_qkv(const dflash_dims *d, const void *wq, const void *wk, const void *wv, void *dst, hipStream_t stream) {
  TRY(check_dims(d, MAX_TARGET_LAYERS));
  TRY(check_ptr(wq, "wq"));
  TRY(check_ptr(wk, "wk"));
  TRY(check_ptr(wv, "wv"));
  TRY(check_ptr(dst, "dst"));
  const int hd = d->head_dim, H = d->hidden;
  const int qr = d->n_q_heads * hd, kr = d->n_kv_heads * hd;
  hipError_t e = launch_pack_matrix(d->dtype, wq, qr, H, dst, 0, 1, hd, qr, false, stream);
  if (e == hipSuccess) e = launch_pack_matrix(d->dtype, wk, kr, H, dst, qr / 16, 1, hd, kr, false, stream);
  if (e == hipSuccess) e = launch_pack_matrix(d->dtype, wv, kr, H, dst, (qr + kr) / 16, 1, hd, 0, false, stream);
  return e == hipSuccess ? DFLASH_OK : hip_fail(e, "pack_qkv");
}

int dflash_pack_gate_up(const dflash_dims *d, const void *wg, const void *wu, void *dst, hipStream_t stream) {
  TRY(check_dims(d, MAX_TARGET_LAYERS));
  TRY(check_ptr(wg, "w_gate"));
  TRY(check_ptr(wu, "w_up"));
  TRY(check_ptr(dst, "dst"));
  const int I = d->intermediate, H = d->hidden;
  hipError_t e = launch_pack_matrix(d->dtype, wg, I, H, dst, 0, 2, 1, 0, true, stream);
  if (e == hipSuccess) e = launch_pack_matrix(d->dtype, wu, I, H, dst, 1, 2, 1, 0, true, stream);
  return e == hipSuccess ? DFLASH_OK : hip_fail(e, "pack_gate_up");
}

size_t dflash_kv_bytes(const dflash_dims *d, int32_t capacity, int32_t max_batch) {
  if (check_dims(d, MAX_TARGET_LAYERS) != DFLASH_OK || capacity <= 0 || max_batch <= 0) return 0;
  return size_t(d->n_layers) * max_batch * d->n_kv_heads * size_t(capacity) * d->head_dim * esize_of(d->dtype);
}

static int kv_convert(const dflash_dims *d, const dflash_kv *kv, void *kp, void *vp, bool to_packed, hipStream_t s) {
  TRY(check_dims(d, MAX_TARGET_LAYERS));
  TRY(check_kv(d, kv));
  TRY(check_ptr(kp, "k_plain"));
  TRY(check_ptr(vp, "v_plain"));
  const long long regions = (long long)d->n_layers * kv->max_batch * d->n_kv_heads;
  const hipError_t e = launch_kv_convert(d->dtype, to_packed, kv->k, kv->v, kp, vp, regions, kv->capacity, d->head_dim, s);
  return e == hipSuccess ? DFLASH_OK : hip_fail(e, "kv convert");
}

int dflash_kv_import(const dflash_dims *d, const dflash_kv *kv, const void *k, const void *v, hipStream_t s) {
  return kv_convert(d, kv, const_cast<void *>(k), const_cast<void *>(v), true, s);
}

int dflash_kv_export(const dflash_dims *d, const dflash_kv *kv, void *k, void *v, hipStream_t s) {
  return kv_convert(d, kv, k, v, false, s);
}

size_t dflash_workspace_bytes(const dflash_dims *d, int32_t max_batch, int32_t max_rows) {
  if (check_dims(d) != DFLASH_OK || max_batch < 1 || max_batch > MAX_BATCH || max_rows < 0) return 0;
  size_t need = draft_layout(d, max_batch).end;
  need = std::max(need, verify_layout(d, max_batch, true).end);
  need = std::max(need, inject_layout(d, std::max(1, max_rows)).end);
  return (need + 255) & ~size_t(255);
}

int dflash_workspace_init(void *ws, size_t bytes, hipStream_t stream) {
  TRY(check_ptr(ws, "ws"));
  if (bytes < WS_COUNTER_BYTES) return fail(DFLASH_ERR_WORKSPACE, "workspace smaller than its counter area");
  const hipError_t e = launch_zero(ws, bytes & ~size_t(15), stream);
  return e == hipSuccess ? DFLASH_OK : hip_fail(e, "workspace_init");
}

int dflash_workspace_view(const dflash_dims *d, int32_t what, int32_t count, int32_t layer, size_t *offset, size_t *bytes) {
  TRY(check_dims(d));
  if (!offset || !bytes) return fail(DFLASH_ERR_NULL, "offset and bytes must be set");
  if (count < 1) return fail(DFLASH_ERR_SHAPE, "count must be >= 1");
  const int H = d->hidden, NQD = d->n_q_heads * d->head_dim;
  if (what == DFLASH_VIEW_FUSED) {
    const InjectLayout L = inject_layout(d, count);
    *offset = L.u;
    *bytes = size_t(count) * H * 4;
    return DFLASH_OK;
  }
  if (count > MAX_BATCH) return fail(DFLASH_ERR_SHAPE, "batch too large");
  const DraftLayout L = draft_layout(d, count);
  const size_t row = size_t(L.M) * H * 4;
  switch (what) {
    case DFLASH_VIEW_HIDDEN:
      if (layer < -1 || layer >= d->n_layers) return fail(DFLASH_ERR_SHAPE, "layer out of range");
      *offset = L.hidden + row * (layer + 1);
      *bytes = row;
      return DFLASH_OK;
    case DFLASH_VIEW_MID:
      if (layer < 0 || layer >= d->n_layers) return fail(DFLASH_ERR_SHAPE, "layer out of range");
      *offset = L.mid + row * layer;
      *bytes = row;
      return DFLASH_OK;
    case DFLASH_VIEW_ATTN:
      if (layer < 0 || layer >= d->n_layers) return fail(DFLASH_ERR_SHAPE, "layer out of range");
      *offset = L.attn + size_t(L.M) * NQD * 4 * layer;
      *bytes = size_t(L.M) * NQD * 4;
      return DFLASH_OK;
    default:
      return fail(DFLASH_ERR_SHAPE, "unknown view");
  }
}

int dflash_inject_kv(const dflash_dims *d, const dflash_weights *w, const dflash_kv *kv, const void *feats,
                     const int32_t *cu_new, int32_t batch, int32_t rows, void *ws, size_t ws_bytes,
                     hipStream_t stream) {
  TRY(check_dims(d));
  TRY(check_weights(d, w, true, false));
  TRY(check_kv(d, kv));
  TRY(check_ptr(cu_new, "cu_new", false));
  TRY(check_ptr(ws, "ws"));
  if (batch < 1 || batch > kv->max_batch) return fail(DFLASH_ERR_SHAPE, "batch must be in [1, kv->max_batch]");
  if (rows < 0) return fail(DFLASH_ERR_SHAPE, "rows must be >= 0");
  if (rows == 0) return DFLASH_OK;
  TRY(check_ptr(feats, "feats"));
  const InjectLayout L = inject_layout(d, rows);
  if (ws_bytes < L.end) return fail(DFLASH_ERR_WORKSPACE, "workspace too small for this many rows");
  char *wsb = static_cast<char *>(ws);
  const int H = d->hidden, kt = kt_of(d->dtype);

  GemmParams fc{};
  fill_gemm(fc, L.fc);
  set_split(fc, wsb, L.part);
  fc.w_seg[0] = static_cast<const char *>(w->w_fc);
  fc.x = static_cast<const char *>(feats);
  fc.x_ld = d->n_feat_layers * H;
  fc.out_f32 = reinterpret_cast<float *>(wsb + L.u);
  fc.ld_out = H;
  float *ssq = reinterpret_cast<float *>(wsb + L.ssq);
  set_norm_out(fc, wsb + L.xc, H / kt, L.xs, L.pc, L.Rp, w->fc_norm, ssq);
  hipError_t e = launch_gemm(d->dtype, EPI_STORE, fc, stream);
  if (e != hipSuccess) return hip_fail(e, "inject fc");

  GemmParams g{};
  fill_gemm(g, L.kv);
  set_split(g, wsb, L.part);
  const int hd = d->head_dim;
  const size_t layer_bytes = packed_bytes(d->dtype, (long long)(d->n_q_heads + 2 * d->n_kv_heads) * hd, H);
  (void)layer_bytes;
  for (int l = 0; l < d->n_layers; ++l)
    g.w_seg[l] = static_cast<const char *>(w->layers[l].w_qkv) + size_t(d->n_q_heads * hd / 16) * (H / kt) * 1024;
  g.seg_ntiles = 2 * d->n_kv_heads * hd / 16;
  g.x = wsb + L.xc;
  g.x_ld = 0;
  g.xs = L.xs;
  g.x_plane = L.pc;
  e = set_norm_in(g, L.rs_inline, ssq, reinterpret_cast<float *>(wsb + L.rs), rows, H, d->rms_eps, stream);
  if (e != hipSuccess) return hip_fail(e, "inject norm");
  g.n_q = d->n_q_heads;
  g.n_kv = d->n_kv_heads;
  g.head_dim = hd;
  fill_rope(g, d);
  g.ctx_len = kv->ctx_len;
  g.kcache = static_cast<char *>(kv->k);
  g.vcache = static_cast<char *>(kv->v);
  g.layer0 = 0;
  g.capacity = kv->capacity;
  g.max_batch = kv->max_batch;
  g.cu_new = cu_new;
  g.batch = batch;
  g.status = kv->status;
  g.arrive = reinterpret_cast<unsigned *>(wsb + WS_ARRIVE_OFFSET);  // the launch commits ctx_len itself
  g.ctx_len_w = kv->ctx_len;
  e = launch_gemm(d->dtype, EPI_KVINJ, g, stream);
  if (e != hipSuccess) return hip_fail(e, "inject kv");
  return DFLASH_OK;
}

// The drafting pass over `batch` blocks: block s holds last_tok[s], then
// mask slots.  Plain form (anchor_pos null): block s is sequence s at its
// frontier.  Anchored form: block s reads cached sequence anchor_seq[s] up to
// position anchor_pos[s] (checked and clamped on the device by the embedding
// launch, which writes the per-block lengths and regions the later launches
// read).
static int draft_impl(const dflash_dims *d, const dflash_weights *w, const dflash_kv *kv, const int32_t *last_tok,
                      const int32_t *anchor_seq, const int32_t *anchor_pos, int32_t batch, int32_t *draft, void *ws,
                      size_t ws_bytes, hipStream_t stream, float temperature = 0.f, const float *u_draft = nullptr,
                      float *draft_logits = nullptr) {
  TRY(check_dims(d));
  TRY(check_weights(d, w, false, true));
  TRY(check_kv(d, kv));
  TRY(check_ptr(last_tok, anchor_pos ? "anchor_tok" : "last_tok", false));
  const bool logits_only = draft_logits && !u_draft;   // draft trees: no per-slot tokens
  if (!logits_only) TRY(check_ptr(draft, "draft", false));
  TRY(check_ptr(ws, "ws"));
  if (anchor_pos) {
    TRY(check_ptr(anchor_seq, "anchor_seq", false));
    if (batch < 1 || batch > MAX_BATCH) return fail(DFLASH_ERR_SHAPE, "nblocks must be in [1, 64]");
  } else if (batch < 1 || batch > kv->max_batch) {
    return fail(DFLASH_ERR_SHAPE, "batch must be in [1, kv->max_batch]");
  }
  const DraftLayout L = draft_layout(d, batch);
  if (ws_bytes < L.end) return fail(DFLASH_ERR_WORKSPACE, "workspace too small for this batch");
  char *wsb = static_cast<char *>(ws);
  const int H = d->hidden, kt = kt_of(d->dtype), hd = d->head_dim, NL = d->n_layers;
  const int NQD = d->n_q_heads * hd, I = d->intermediate;
  const size_t row = size_t(L.M) * H * 4;
  float *hidden = reinterpret_cast<float *>(wsb + L.hidden);
  float *mid = reinterpret_cast<float *>(wsb + L.mid);
  const size_t region_layer = size_t(kv->max_batch) * d->n_kv_heads * size_t(kv->capacity) * hd * esize_of(d->dtype);
  float *ssq = reinterpret_cast<float *>(wsb + L.ssq);
  float *rs = reinterpret_cast<float *>(wsb + L.rs);
  hipError_t e;

  // Every RMSNorm is split: its producer (the embedding, o_proj, down) writes
  // the rows * gain into xa plus tile sums of squares; its consumer (QKV,
  // gate_up, lm_head) scales its output rows by 1 / rms.
  EmbedParams ep{};
  ep.embed = static_cast<const char *>(w->embed);
  ep.last_tok = last_tok;
  ep.block = d->block_size;
  ep.mask_id = d->mask_id;
  ep.vocab = d->vocab;
  ep.status = kv->status;
  ep.gathered = hidden;
  ep.gain = static_cast<const char *>(w->layers[0].attn_norm);
  ep.M = L.M;
  ep.rows_pad = L.Mp;
  ep.H = H;
  ep.xpacked = wsb + L.xa;
  ep.x_kt = H / kt;
  ep.planes = L.xs;
  ep.x_plane = L.pa;
  ep.ssq = ssq;
  int *blk_ctx = reinterpret_cast<int *>(wsb + L.anc), *blk_region = blk_ctx + MAX_BATCH;
  if (anchor_pos) {
    ep.anchor_seq = anchor_seq;
    ep.anchor_pos = anchor_pos;
    ep.ctx_len = kv->ctx_len;
    ep.max_batch = kv->max_batch;
    ep.capacity = kv->capacity;
    ep.blk_ctx = blk_ctx;
    ep.blk_region = blk_region;
  }
  // the context each block attends to (and its rotary base position)
  const int *ctx_of = anchor_pos ? blk_ctx : kv->ctx_len;
  e = launch_embed(d->dtype, ep, stream);
  if (e != hipSuccess) return hip_fail(e, "draft embed");

  LayerRun run{};
  run.d = d;
  run.L = &L;
  run.wsb = wsb;
  run.batch = batch;
  run.ctx_of = ctx_of;
  run.region_of = anchor_pos ? blk_region : nullptr;
  run.kcache = static_cast<const char *>(kv->k);
  run.vcache = static_cast<const char *>(kv->v);
  run.region_layer = region_layer;
  run.capacity = kv->capacity;
  run.max_batch = kv->max_batch;
  run.status = kv->status;
  run.what = "draft";
  for (int l = 0; l < NL; ++l) {
    float *h_in = reinterpret_cast<float *>(reinterpret_cast<char *>(hidden) + row * l);
    float *h_mid = reinterpret_cast<float *>(reinterpret_cast<char *>(mid) + row * l);
    float *h_out = reinterpret_cast<float *>(reinterpret_cast<char *>(hidden) + row * (l + 1));
    float *attn_out = reinterpret_cast<float *>(wsb + L.attn + size_t(L.M) * NQD * 4 * l);
    const void *next_gain = l + 1 < NL ? w->layers[l + 1].attn_norm : w->final_norm;
    TRY(run_layer(run, w->layers[l], l, next_gain, h_in, h_mid, h_out, attn_out, nullptr, 0, stream));
  }

  GemmParams lm{};
  fill_gemm(lm, L.lm);
  lm.w_seg[0] = static_cast<const char *>(w->lm_head);
  lm.x = wsb + L.xa;
  // The head reads the hi plane only: the normalised hidden rounded to bf16
  // moves a logit by ~1e-3 (std), an order below the 1e-2 gap at which a
  // drafted token is decided, and halves the head's MFMA work.
  lm.xs = 1;
  lm.x_plane = L.pa;
  e = set_norm_in(lm, L.rs_inline, ssq, rs, L.M, H, d->rms_eps, stream);
  if (e != hipSuccess) return hip_fail(e, "draft final norm");
  lm.vocab = d->vocab;
  lm.keys = reinterpret_cast<unsigned long long *>(wsb);
  ArgmaxFinishParams fp{};
  fp.keys = lm.keys;
  fp.rows_per_seq = d->block_size;
  fp.block = d->block_size;
  fp.verify = 0;
  fp.tok_out = draft;
  if (temperature <= 0.f && !draft_logits) return launch_argmax_head(d->dtype, lm, fp, wsb, batch, stream, "draft");
  // Sampling (and draft trees): the head stores its logits; for sampling a
  // Gumbel-max per row, folded by the argmax finish.
  lm.out_f32 = draft_logits;
  lm.ld_out = d->vocab;
  e = launch_gemm(d->dtype, EPI_LOGITS, lm, stream);
  if (e != hipSuccess) return hip_fail(e, "draft logits");
  if (!u_draft) return DFLASH_OK;
  SampleParams sp{};
  sp.logits = draft_logits;
  sp.ld = d->vocab;
  sp.vocab = d->vocab;
  sp.chunks = sample_chunks(d->vocab);
  sp.inv_t = 1.0f / temperature;
  sp.u = u_draft;
  sp.keys = lm.keys;
  e = launch_gumbel_draft(sp, L.M, stream);
  if (e == hipSuccess) e = launch_argmax_finish(fp, batch, stream);
  return e == hipSuccess ? DFLASH_OK : hip_fail(e, "draft sampling");
}

int dflash_draft_forward(const dflash_dims *d, const dflash_weights *w, const dflash_kv *kv, const int32_t *last_tok,
                         int32_t batch, int32_t *draft, void *ws, size_t ws_bytes, hipStream_t stream) {
  return draft_impl(d, w, kv, last_tok, nullptr, nullptr, batch, draft, ws, ws_bytes, stream);
}

int dflash_draft_anchors(const dflash_dims *d, const dflash_weights *w, const dflash_kv *kv, const int32_t *anchor_seq,
                         const int32_t *anchor_pos, const int32_t *anchor_tok, int32_t nblocks, int32_t *draft,
                         void *ws, size_t ws_bytes, hipStream_t stream) {
  TRY(check_ptr(anchor_pos, "anchor_pos", false));
  return draft_impl(d, w, kv, anchor_tok, anchor_seq, anchor_pos, nblocks, draft, ws, ws_bytes, stream);
}

size_t dflash_target_workspace_bytes(const dflash_dims *td, int32_t max_batch, int32_t rows) {
  if (check_dims(td, MAX_TARGET_LAYERS) != DFLASH_OK || max_batch < 1 || max_batch > MAX_BATCH || rows < 1 ||
      rows > 32)
    return 0;
  return (draft_layout(td, max_batch, rows, true).end + 255) & ~size_t(255);
}

int dflash_target_forward(const dflash_dims *td, const dflash_weights *tw, const dflash_kv *tkv,
                          const int32_t *tokens, const int32_t *parents, int32_t batch, int32_t rows,
                          const int32_t *feat_layers, int32_t n_feat, void *out_hidden, void *out_feats, void *ws,
                          size_t ws_bytes, hipStream_t stream) {
  TRY(check_dims(td, MAX_TARGET_LAYERS));
  if (!tw) return fail(DFLASH_ERR_NULL, "weights is NULL");
  if (!tw->layers) return fail(DFLASH_ERR_NULL, "weights->layers is NULL");
  TRY(check_ptr(tw->embed, "embed"));
  TRY(check_ptr(tw->final_norm, "final_norm"));
  for (int l = 0; l < td->n_layers; ++l) {
    const dflash_layer &L = tw->layers[l];
    TRY(check_ptr(L.attn_norm, "layers[].attn_norm"));
    TRY(check_ptr(L.w_qkv, "layers[].w_qkv"));
    TRY(check_ptr(L.w_o, "layers[].w_o"));
    TRY(check_ptr(L.mlp_norm, "layers[].mlp_norm"));
    TRY(check_ptr(L.w_gate_up, "layers[].w_gate_up"));
    TRY(check_ptr(L.w_down, "layers[].w_down"));
  }
  TRY(check_kv(td, tkv));
  TRY(check_ptr(tokens, "tokens", false));
  TRY(check_ptr(out_hidden, "out_hidden", false));
  TRY(check_ptr(ws, "ws"));
  if (batch < 1 || batch > tkv->max_batch) return fail(DFLASH_ERR_SHAPE, "batch must be in [1, kv->max_batch]");
  // the block's K/V are one key step of the attention: 32 rows (bf16), 16 (fp32)
  if (rows < 1 || rows > kt_of(td->dtype))
    return fail(DFLASH_ERR_SHAPE, "rows must be in [1, 32] (bf16) or [1, 16] (fp32)");
  if (n_feat < 0 || n_feat > 16) return fail(DFLASH_ERR_SHAPE, "n_feat must be in [0, 16]");
  if (n_feat > 0) {
    TRY(check_ptr(feat_layers, "feat_layers", false));
    TRY(check_ptr(out_feats, "out_feats", false));
    for (int k = 0; k < n_feat; ++k) {
      if (feat_layers[k] < 0 || feat_layers[k] >= td->n_layers)
        return fail(DFLASH_ERR_SHAPE, "feat_layers entries must lie in [0, n_layers)");
      for (int k2 = 0; k2 < k; ++k2)
        if (feat_layers[k2] == feat_layers[k]) return fail(DFLASH_ERR_SHAPE, "feat_layers entries must be distinct");
    }
  }
  const DraftLayout L = draft_layout(td, batch, rows, true);
  if (ws_bytes < L.end) return fail(DFLASH_ERR_WORKSPACE, "workspace too small (dflash_target_workspace_bytes)");
  char *wsb = static_cast<char *>(ws);
  const int H = td->hidden, kt = kt_of(td->dtype), es = esize_of(td->dtype);
  const size_t row = size_t(L.M) * H * 4;
  float *hbuf[2] = {reinterpret_cast<float *>(wsb + L.hidden), reinterpret_cast<float *>(wsb + L.hidden + row)};
  float *mid = reinterpret_cast<float *>(wsb + L.mid);
  float *attn_out = reinterpret_cast<float *>(wsb + L.attn);

  EmbedParams ep{};
  ep.embed = static_cast<const char *>(tw->embed);
  ep.tokens = tokens;
  ep.block = rows;
  ep.vocab = td->vocab;
  ep.status = tkv->status;
  ep.gathered = hbuf[0];
  ep.gain = static_cast<const char *>(tw->layers[0].attn_norm);
  ep.M = L.M;
  ep.rows_pad = L.Mp;
  ep.H = H;
  ep.xpacked = wsb + L.xa;
  ep.x_kt = H / kt;
  ep.planes = L.xs;
  ep.x_plane = L.pa;
  ep.ssq = reinterpret_cast<float *>(wsb + L.ssq);
  hipError_t e = launch_embed(td->dtype, ep, stream);
  if (e != hipSuccess) return hip_fail(e, "target embed");

  LayerRun run{};
  run.d = td;
  run.L = &L;
  run.wsb = wsb;
  run.batch = batch;
  run.ctx_of = tkv->ctx_len;
  run.kcache = static_cast<const char *>(tkv->k);
  run.vcache = static_cast<const char *>(tkv->v);
  run.region_layer = size_t(tkv->max_batch) * td->n_kv_heads * size_t(tkv->capacity) * td->head_dim * es;
  run.capacity = tkv->capacity;
  run.max_batch = tkv->max_batch;
  run.causal = true;
  run.status = tkv->status;
  run.what = "target";
  if (parents) {
    int *depth = reinterpret_cast<int *>(wsb + L.tree);
    unsigned *mask = reinterpret_cast<unsigned *>(depth + L.M);
    e = launch_tree_prep(parents, batch, rows, depth, mask, tkv->status, stream);
    if (e != hipSuccess) return hip_fail(e, "target tree");
    run.row_pos = depth;
    run.row_mask = mask;
  }
  const int NL = td->n_layers;
  for (int l = 0; l < NL; ++l) {
    char *aux = nullptr;   // feature k: columns [k H, (k + 1) H) of out_feats
    for (int k = 0; k < n_feat; ++k)
      if (feat_layers[k] == l) aux = static_cast<char *>(out_feats) + size_t(k) * H * es;
    const void *next_gain = l + 1 < NL ? tw->layers[l + 1].attn_norm : tw->final_norm;
    TRY(run_layer(run, tw->layers[l], l, next_gain, hbuf[l & 1], mid, hbuf[(l + 1) & 1], attn_out, aux,
                  n_feat * H, stream));
  }
  e = launch_rownorm(td->dtype, hbuf[NL & 1], L.M, H, tw->final_norm, td->rms_eps, out_hidden, stream);
  return e == hipSuccess ? DFLASH_OK : hip_fail(e, "target final norm");
}

int dflash_kv_commit(const dflash_dims *d, const dflash_kv *kv, const int32_t *accept_len, int32_t batch,
                     int32_t max_commit, hipStream_t stream) {
  TRY(check_dims(d, MAX_TARGET_LAYERS));
  TRY(check_kv(d, kv));
  TRY(check_ptr(accept_len, "accept_len", false));
  if (batch < 1 || batch > kv->max_batch) return fail(DFLASH_ERR_SHAPE, "batch must be in [1, kv->max_batch]");
  if (max_commit < 0) return fail(DFLASH_ERR_SHAPE, "max_commit must be >= 0");
  const hipError_t e = launch_kv_commit(kv->ctx_len, accept_len, batch, max_commit, kv->capacity, stream);
  return e == hipSuccess ? DFLASH_OK : hip_fail(e, "kv commit");
}

int dflash_draft_tree(const dflash_dims *d, const dflash_weights *w, const dflash_kv *kv, const int32_t *last_tok,
                      int32_t batch, int32_t topk, int32_t nodes, float *draft_logits, int32_t *tree_tok,
                      int32_t *tree_parent, void *ws, size_t ws_bytes, hipStream_t stream) {
  TRY(check_dims(d));
  if (batch < 1 || batch > MAX_BATCH) return fail(DFLASH_ERR_SHAPE, "batch must be in [1, 64]");
  if (topk < 1 || topk > 8) return fail(DFLASH_ERR_SHAPE, "topk must be in [1, 8]");
  if (nodes < 1 || nodes > 31) return fail(DFLASH_ERR_SHAPE, "nodes must be in [1, 31]");
  long long avail = 0, pw = 1;   // continuations of length 1 .. B over topk tokens per slot
  for (int j = 0; j < d->block_size && avail < nodes; ++j) {
    pw *= topk;
    avail += pw;
  }
  if (avail < nodes) return fail(DFLASH_ERR_SHAPE, "nodes exceeds the continuations of block_size slots over topk tokens");
  TRY(check_ptr(draft_logits, "draft_logits", false));
  TRY(check_ptr(tree_tok, "tree_tok", false));
  TRY(check_ptr(tree_parent, "tree_parent", false));
  // the drafting pass with its logits (placeholder draft output: the tree
  // replaces the per-slot tokens)
  const DraftLayout L = draft_layout(d, batch);
  if (!ws || ws_bytes < L.end) return fail(DFLASH_ERR_WORKSPACE, "workspace too small for this batch");
  TRY(draft_impl(d, w, kv, last_tok, nullptr, nullptr, batch, nullptr, ws, ws_bytes, stream, 1.0f, nullptr,
                 draft_logits));
  char *wsb = static_cast<char *>(ws);
  const int V = d->vocab, rows = L.M, ch = sample_chunks(V);
  float *lse = reinterpret_cast<float *>(wsb + L.tree);
  float2 *part = reinterpret_cast<float2 *>(lse + rows);
  float *tv = reinterpret_cast<float *>(part + size_t(rows) * ARGMAX_SLOTS);
  int *ti = reinterpret_cast<int *>(tv + size_t(rows) * 8);
  auto *ck = reinterpret_cast<unsigned long long *>(ti + size_t(rows) * 8);
  hipError_t e = launch_row_lse(draft_logits, V, V, 1.0f, rows, ch, part, lse, stream);
  if (e == hipSuccess) e = launch_row_topk(draft_logits, V, V, rows, topk, lse, ck, tv, ti, stream);
  if (e == hipSuccess)
    e = launch_tree_build(tv, ti, last_tok, batch, d->block_size, topk, nodes, tree_tok, tree_parent, stream);
  return e == hipSuccess ? DFLASH_OK : hip_fail(e, "draft tree");
}

int dflash_tree_accept(const dflash_dims *d, const void *lm_head, const void *target_hidden, const int32_t *tree_tok,
                       const int32_t *tree_parent, int32_t batch, int32_t n, int32_t *target_argmax,
                       int32_t *accept_len, int32_t *bonus, int32_t *path, void *ws, size_t ws_bytes,
                       hipStream_t stream) {
  TRY(check_dims(d));
  TRY(check_ptr(lm_head, "lm_head"));
  TRY(check_ptr(target_hidden, "target_hidden"));
  TRY(check_ptr(tree_tok, "tree_tok", false));
  TRY(check_ptr(tree_parent, "tree_parent", false));
  TRY(check_ptr(target_argmax, "target_argmax", false));
  TRY(check_ptr(accept_len, "accept_len", false));
  TRY(check_ptr(bonus, "bonus", false));
  TRY(check_ptr(path, "path", false));
  TRY(check_ptr(ws, "ws"));
  if (batch < 1 || batch > MAX_BATCH) return fail(DFLASH_ERR_SHAPE, "batch must be in [1, 64]");
  if (n < 1 || n > 32 || size_t(batch) * n > size_t(MAX_KEY_ROWS)) return fail(DFLASH_ERR_SHAPE, "n must be in [1, 32]");
  if (ws_bytes < WS_COUNTER_BYTES) return fail(DFLASH_ERR_WORKSPACE, "workspace smaller than its counter area");
  char *wsb = static_cast<char *>(ws);
  GemmParams lm{};
  fill_gemm(lm, plan_head(d->dtype, batch * n, d->vocab, d->hidden));
  lm.w_seg[0] = static_cast<const char *>(lm_head);
  lm.x = static_cast<const char *>(target_hidden);
  lm.x_ld = d->hidden;
  lm.vocab = d->vocab;
  lm.keys = reinterpret_cast<unsigned long long *>(wsb);
  ArgmaxFinishParams fp{};
  fp.keys = lm.keys;
  fp.rows_per_seq = n;
  fp.block = n;
  fp.verify = 0;
  fp.tok_out = target_argmax;
  TRY(launch_argmax_head(d->dtype, lm, fp, wsb, batch, stream, "tree verify"));
  const hipError_t e = launch_tree_walk(tree_tok, tree_parent, target_argmax, batch, n, accept_len, bonus, path, stream);
  return e == hipSuccess ? DFLASH_OK : hip_fail(e, "tree walk");
}

int dflash_kv_commit_path(const dflash_dims *d, const dflash_kv *kv, const int32_t *path, const int32_t *accept_len,
                          int32_t batch, int32_t n, hipStream_t stream) {
  TRY(check_dims(d, MAX_TARGET_LAYERS));
  TRY(check_kv(d, kv));
  TRY(check_ptr(path, "path", false));
  TRY(check_ptr(accept_len, "accept_len", false));
  if (batch < 1 || batch > kv->max_batch) return fail(DFLASH_ERR_SHAPE, "batch must be in [1, kv->max_batch]");
  if (n < 1 || n > 32) return fail(DFLASH_ERR_SHAPE, "n must be in [1, 32]");
  const hipError_t e = launch_commit_path(d->dtype, static_cast<char *>(kv->k), static_cast<char *>(kv->v), kv->ctx_len,
                                          path, accept_len, batch, n, d->n_layers, kv->max_batch, d->n_kv_heads,
                                          kv->capacity, d->head_dim, stream);
  return e == hipSuccess ? DFLASH_OK : hip_fail(e, "kv commit path");
}

int dflash_draft_sample(const dflash_dims *d, const dflash_weights *w, const dflash_kv *kv, const int32_t *last_tok,
                        int32_t batch, float temperature, const float *u_draft, int32_t *draft, float *draft_logits,
                        void *ws, size_t ws_bytes, hipStream_t stream) {
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(DFLASH_ERR_SHAPE, "temperature must be positive and finite (greedy drafting: dflash_draft_forward)");
  TRY(check_ptr(u_draft, "u_draft", false));
  TRY(check_ptr(draft_logits, "draft_logits", false));
  return draft_impl(d, w, kv, last_tok, nullptr, nullptr, batch, draft, ws, ws_bytes, stream, temperature, u_draft,
                    draft_logits);
}

int dflash_verify_sample(const dflash_dims *d, const void *lm_head, const void *target_hidden, const int32_t *draft,
                         const float *draft_logits, int32_t batch, float temperature, const float *u_accept,
                         const float *u_resid, float *target_logits, int32_t *accept_len, int32_t *next_tok,
                         void *ws, size_t ws_bytes, hipStream_t stream) {
  TRY(check_dims(d));
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(DFLASH_ERR_SHAPE, "temperature must be positive and finite (greedy verification: dflash_verify_accept)");
  TRY(check_ptr(lm_head, "lm_head"));
  TRY(check_ptr(target_hidden, "target_hidden"));
  TRY(check_ptr(draft, "draft", false));
  TRY(check_ptr(draft_logits, "draft_logits", false));
  TRY(check_ptr(u_accept, "u_accept", false));
  TRY(check_ptr(u_resid, "u_resid", false));
  TRY(check_ptr(target_logits, "target_logits", false));
  TRY(check_ptr(accept_len, "accept_len", false));
  TRY(check_ptr(next_tok, "next_tok", false));
  TRY(check_ptr(ws, "ws"));
  if (batch < 1 || batch > MAX_BATCH) return fail(DFLASH_ERR_SHAPE, "batch must be in [1, 64]");
  const VerifyLayout L = verify_layout(d, batch, true);
  if (ws_bytes < L.end) return fail(DFLASH_ERR_WORKSPACE, "workspace too small for this batch");
  char *wsb = static_cast<char *>(ws);
  const int B = d->block_size, V = d->vocab;
  GemmParams lm{};
  fill_gemm(lm, L.lm);
  lm.w_seg[0] = static_cast<const char *>(lm_head);
  lm.x = static_cast<const char *>(target_hidden);
  lm.x_ld = d->hidden;
  lm.vocab = V;
  lm.out_f32 = target_logits;
  lm.ld_out = V;
  hipError_t e = launch_gemm(d->dtype, EPI_LOGITS, lm, stream);
  if (e != hipSuccess) return hip_fail(e, "verify logits");
  const float inv_t = 1.0f / temperature;
  float *lse_q = reinterpret_cast<float *>(wsb + L.lse), *lse_p = lse_q + size_t(batch) * B;
  float2 *part = reinterpret_cast<float2 *>(wsb + L.lse_part);
  const int ch = sample_chunks(V);
  e = launch_row_lse(draft_logits, V, V, inv_t, batch * B, ch, part, lse_q, stream);
  if (e == hipSuccess)
    e = launch_row_lse(target_logits, V, V, inv_t, batch * (B + 1), ch, part + size_t(batch) * B * ch, lse_p, stream);
  if (e != hipSuccess) return hip_fail(e, "verify log-sum-exp");
  SampleParams sp{};
  sp.ld = V;
  sp.vocab = V;
  sp.chunks = sample_chunks(V);
  sp.inv_t = inv_t;
  sp.keys = reinterpret_cast<unsigned long long *>(wsb);
  sp.q_logits = draft_logits;
  sp.p_logits = target_logits;
  sp.lse_q = lse_q;
  sp.lse_p = lse_p;
  sp.draft = draft;
  sp.block = B;
  sp.u_accept = u_accept;
  sp.u_resid = u_resid;
  sp.accept_len = accept_len;
  e = launch_spec_sample(sp, batch, stream);
  ArgmaxFinishParams fp{};
  fp.keys = sp.keys;
  fp.rows_per_seq = 1;
  fp.block = 1;
  fp.verify = 0;
  fp.tok_out = next_tok;
  if (e == hipSuccess) e = launch_argmax_finish(fp, batch, stream);
  return e == hipSuccess ? DFLASH_OK : hip_fail(e, "verify sampling");
}

int dflash_verify_accept(const dflash_dims *d, const void *lm_head, const void *target_hidden, const int32_t *draft,
                         int32_t batch, int32_t *target_argmax, int32_t *accept_len, int32_t *bonus, void *ws,
                         size_t ws_bytes, hipStream_t stream) {
  TRY(check_ptr(ws, "ws"));
  return verify_with_ws(d, lm_head, target_hidden, draft, batch, target_argmax, accept_len, bonus,
                        static_cast<char *>(ws), ws_bytes, stream);
}

}  // extern "C"
