// Y = X W^T on MFMA for the skinny shapes of a draft step (16 rows per
// sequence), with fused epilogues.
//
// Operands are packed fragment tiles (1 KiB = one 64-lane MFMA operand), so
// every wavefront load is a single coalesced 1 KiB read.  The weight tile is
// the A operand (rows = output features) and the activation tile the B
// operand (rows = tokens); lane (c, g) of an accumulator then holds token c
// and output features 4g..4g+3.
//
// A workgroup owns NB 16-column weight tiles for MT 16-row token tiles and the
// whole K range.  Its 8 wavefronts split K, stream their weight tiles
// with non-temporal loads, and add their partial tiles in LDS in a fixed
// order, so the result does not depend on scheduling and no workgroup ever
// waits on another.  The epilogue runs in the same workgroup.  The vocabulary
// argmax is the one cross-workgroup reduction: each workgroup folds its best
// (logit, index) key per row into one of 64 slots with a 64-bit atomic max,
// and a small follow-up kernel reads the slots after the kernel boundary.
#include "common.hpp"
#include "kernels.hpp"
#include "gemm_util.hpp"

namespace dflash {

__device__ inline float tile_at(const f32x4 *t, int NB, int ml, int nl) {
  const int f = (ml >> 4) * NB + (nl >> 4);
  const int ln = (ml & 15) + 16 * ((nl & 15) >> 2);
  return t[f * 64 + ln][nl & 3];
}

// Every GEMM workgroup has 8 wavefronts (two per SIMD, so each may hold up to
// 256 VGPRs) and deals the k-tiles out to them round-robin (wavefront w takes
// w, w + 8, ...) whatever the row-tile count.  A wavefront consumes its share
// in batches (of four for one-tile items of one row tile, else two); even and odd k-tiles feed two accumulator
// chains per activation plane (one chain per plane when NB * XS >= 4); chains
// and wavefronts are summed in a fixed order.  The summation order of a row therefore never depends on how
// many other rows share the launch.
constexpr int GEMM_WAVES = 8;
// 17-row launches (X1): most k-tiles a wavefront's chunk may hold (K <= 12288 for bf16)
constexpr int X1_MAX_KTILES = 48;
// LDS staging of an inline RMSNorm's tile sums: rows x tiles <= 8192 floats.
constexpr int RS_STAGE_FLOATS = 8192;
constexpr int GEMM_THREADS = GEMM_WAVES * 64;
// k-tiles per batch: 4 (a wavefront keeps 8 or 16 KiB of weights in flight
// over its two batches) unless the streamed activations of MT = 4 row tiles
// would not fit; then 2.
template <int MT, int NB> constexpr int gemm_u() { return MT <= (NB == 1 ? 1 : 2) ? 4 : 2; }

template <int U, int NB> struct WBatch { uint4 w[U][NB]; };
template <int U, int MT, int NB, int XS> struct XWBatch {
  uint4 w[U][NB];
  uint4 x[U][MT][XS];
};

// Epilogue of one output tile (the reduced MT x NB fragment tile in LDS).
// rs: per-row scales of the activations' RMSNorm (nullptr: none).
template <typename T, int MT, int NB, int EPI>
__device__ inline void gemm_epilogue(const GemmParams &p, const f32x4 *red, const float *rs, int mblk, int nblk,
                                     unsigned long long *best_row) {
  constexpr int KT = Ty<T>::KT, ES = Ty<T>::SIZE;
  constexpr int R = MT * 16, CN = NB * 16, NT = GEMM_THREADS;
  auto val = [&](int ml, int nl) { return rs ? tile_at(red, NB, ml, nl) * rs[ml] : tile_at(red, NB, ml, nl); };
  // columns nl0 .. nl0 + 3 (nl0 a multiple of 4: one f32x4 of the tile)
  auto val4 = [&](int ml, int nl0) {
    const f32x4 t = red[((ml >> 4) * NB + (nl0 >> 4)) * 64 + (ml & 15) + 16 * ((nl0 & 15) >> 2)];
    return rs ? t * rs[ml] : t;
  };
  if constexpr (EPI == EPI_STORE || EPI == EPI_RESID) {
    // 16 consecutive threads hold one row of the 16-column tile, so the
    // tile's sum of squares is one butterfly (tile_ssq16).  The residual and
    // the gain are loaded before any store (a load behind a store waits for
    // it).
    static_assert(CN == 16, "row-major epilogues take one 16-column tile");
    for (int e = threadIdx.x; e < R * CN; e += NT) {
      const int ml = e / CN, nl = e % CN;
      const int m = mblk * R + ml, n = nblk * CN + nl;
      const bool ok = m < p.M && n < p.N;
      const bool nx = p.nx_packed && n < p.N && m < p.nx_rows;
      const size_t o = size_t(m) * p.ld_out + n;
      float v = 0.f;
      if constexpr (EPI == EPI_RESID) {
        if (ok) v = p.resid[o];
      }
      const float gain = nx ? to_f32<T>(reinterpret_cast<const T *>(p.nx_gain)[n]) : 0.f;
      if (ok) {
        v = EPI == EPI_RESID ? val(ml, nl) + v : val(ml, nl);
        p.out_f32[o] = v;
        if (p.aux_out) store_elem<T>(p.aux_out + (size_t(m) * p.aux_ld + n) * ES, v);
      }
      if (nx) store_split<T>(p.nx_packed + packed_offset<T>(m, n, p.nx_kt), p.nx_plane, p.nx_planes, v * gain);
      if (p.ssq_out) {
        const float t = tile_ssq16(v);
        if (nl == 0 && ok) p.ssq_out[size_t(m) * p.ssq_ld + nblk] = t;
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    // four consecutive columns per thread: one store per plane
    constexpr int HALF = NB / 2;
    for (int e = threadIdx.x; e < R * HALF * 4; e += NT) {
      const int ml = e / (HALF * 4), q = e % (HALF * 4);
      const int pr = q >> 2, c4 = 4 * (q & 3);
      const int m = mblk * R + ml;  // padded rows get zeros
      f32x4 out = f32x4{0.f, 0.f, 0.f, 0.f};
      if (m < p.M) {
        const f32x4 gt = val4(ml, 2 * pr * 16 + c4), up = val4(ml, (2 * pr + 1) * 16 + c4);
#pragma unroll
        for (int i = 0; i < 4; ++i) out[i] = gt[i] / (1.0f + __expf(-gt[i])) * up[i];
      }
      store_split4<T>(p.out_packed + packed_offset<T>(m, (nblk * HALF + pr) * 16 + c4, p.out_kt), p.out_plane,
                      p.out_planes, out);
    }
  } else if constexpr (EPI == EPI_QKV) {
    const int d = p.head_dim, nqd = p.n_q * d, nkd = p.n_kv * d;
    const int dt_count = d / KT;
    for (int e = threadIdx.x; e < R * CN; e += NT) {
      const int ml = e / CN, nl = e % CN;
      const int m = mblk * R + ml, n = nblk * CN + nl;
      if (m >= p.M) continue;
      const int s = m / p.block, j = m % p.block;
      float v = val(ml, nl);
      if (n < nqd + nkd) {
        const int dd = rot_channel(n % d, d);
        const int pos = p.ctx_len[s] + (p.row_pos ? p.row_pos[m] : j);
        v = rope_apply(v, val(ml, nl ^ 8), dd, d, pos, p);
        if (n < nqd) {
          const int h = n / d;
          char *base = p.qbuf + (size_t(s) * p.n_q + h) * p.q_tiles * dt_count * 1024;
          store_split<T>(base + packed_offset<T>(j, dd, dt_count), p.q_plane, p.q_planes, v);
        } else {
          const int g = (n - nqd) / d;
          char *base = p.kblk + (size_t(s) * p.n_kv + g) * size_t(KT) * d * ES;
          store_elem<T>(base + kcache_offset<T>(j, dd, d), v);
          // cache slot ctx + j (slot order); its rotary position may be a tree depth
          if (p.qkv_to_cache) qkv_cache_store<T>(p, true, s, g, p.ctx_len[s] + j, dd, v);
        }
      } else {
        const int c = n - nqd - nkd;
        const int g = c / d, dd = c % d;
        char *base = p.vblk + (size_t(s) * p.n_kv + g) * size_t(KT) * d * ES;
        store_elem<T>(base + vcache_offset<T>(j, dd, d), v);
        if (p.qkv_to_cache) qkv_cache_store<T>(p, false, s, g, p.ctx_len[s] + j, dd, v);
      }
    }
  } else if constexpr (EPI == EPI_KVINJ) {
    const int d = p.head_dim, nkd = p.n_kv * d, segn = 2 * nkd;
    const size_t region = size_t(p.capacity) * d * ES;
    for (int e = threadIdx.x; e < R * CN; e += NT) {
      const int ml = e / CN, nl = e % CN;
      const int m = mblk * R + ml, n = nblk * CN + nl;
      if (m >= p.M) continue;
      int lo = 0, hi = p.batch;  // find s with cu_new[s] <= m < cu_new[s+1]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.cu_new[mid] <= m) lo = mid; else hi = mid;
      }
      const int s = lo, start = p.cu_new[s], ns = p.cu_new[s + 1] - start;
      const int C = p.ctx_len[s];
      if (C + ns > p.capacity) {
        if (m == start && n == 0) atomicOr(p.status, DFLASH_STATUS_CAPACITY);
        continue;
      }
      const int pos = C + (m - start);
      const int layer = p.layer0 + n / segn, c = n % segn;
      const float v = val(ml, nl);
      if (c < nkd) {
        const int g = c / d, dd = rot_channel(c % d, d);
        const float r = rope_apply(v, val(ml, nl ^ 8), dd, d, pos, p);
        char *base = p.kcache + ((size_t(layer) * p.max_batch + s) * p.n_kv + g) * region;
        store_elem<T>(base + kcache_offset<T>(pos, dd, d), r);
      } else {
        const int c2 = c - nkd, g = c2 / d, dd = c2 % d;
        char *base = p.vcache + ((size_t(layer) * p.max_batch + s) * p.n_kv + g) * region;
        store_elem<T>(base + vcache_offset<T>(pos, dd, d), v);
      }
    }
  } else if constexpr (EPI == EPI_LOGITS) {
    for (int e = threadIdx.x; e < R * CN; e += NT) {
      const int ml = e / CN, nl = e % CN;
      const int m = mblk * R + ml, n = nblk * CN + nl;
      if (m < p.M && n < p.vocab) p.out_f32[size_t(m) * p.ld_out + n] = val(ml, nl);
    }
  } else if constexpr (EPI == EPI_ARGMAX) {
    // Running best (logit, index) key per row over this workgroup's tiles:
    // one element per thread, a 32-lane shuffle max per row (CN == 32), and
    // the row's leader folds the result into best_row.
    static_assert(CN == 32, "argmax epilogue expects 32 columns per tile");
    for (int e0 = 0; e0 < R * CN; e0 += NT) {
      const int e = e0 + int(threadIdx.x);
      const int ml = e >> 5, nl = e & 31;
      const int n = nblk * CN + nl;
      unsigned long long k = 0;
      if (ml < R && n < p.vocab) k = argmax_key(val(ml, nl), n);
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) {
        const unsigned long long o = __shfl_xor(k, off, 64);
        k = o > k ? o : k;
      }
      if (nl == 0 && ml < R && k > best_row[ml]) best_row[ml] = k;
    }
  }
}

// Argmax finish for at most FUSED_FINISH_ROWS rows, run by one workgroup of
// GEMM_THREADS threads after every workgroup's slot updates are performed:
// 8 threads per row read and clear 8 slots each with atomic exchanges, fold
// them by an 8-lane shuffle max, then one thread per sequence runs the
// acceptance scan (verify).
__device__ inline void fused_argmax_finish(const ArgmaxFinishParams &f, int M, int *toks) {
  const int row = threadIdx.x >> 3, q = threadIdx.x & 7;
  unsigned long long best = 0;
  if (row < M) {
    unsigned long long *k = f.keys + size_t(row) * ARGMAX_SLOTS + q * (ARGMAX_SLOTS / 8);
#pragma unroll
    for (int i = 0; i < ARGMAX_SLOTS / 8; ++i) {
      const unsigned long long v = __hip_atomic_exchange(k + i, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      best = v > best ? v : best;
    }
  }
#pragma unroll
  for (int off = 1; off < 8; off <<= 1) {
    const unsigned long long o = __shfl_xor(best, off, 64);
    best = o > best ? o : best;
  }
  if (row < M && q == 0) {
    const int tok = key_index(best);
    f.tok_out[row] = tok;
    toks[row] = tok;
  }
  __syncthreads();
  if (f.verify) {
    const int R = f.rows_per_seq, B = f.block;
    const int s = threadIdx.x;
    if (s < M / R) {
      int L = B;
      for (int j = 0; j < B; ++j) {
        if (f.draft_in[s * B + j] != toks[s * R + j]) { L = j; break; }
      }
      f.accept_len[s] = L;
      f.bonus[s] = toks[s * R + L];
    }
  }
}

// XROW: activations are a row-major [M, x_ld] input (one plane); otherwise
// packed fragment tiles padded to whole row blocks (so no load needs a guard).
// KC > 0: every wavefront's K chunk (at most KC tiles) of activations is
// loaded into registers once, and only weights stream through the loop (the
// texture-address unit, not HBM, limits a loop that also streams
// activations).  KC == 0: activations stream with the weights.
//
// RMSNorm: the activations arrive as (x * gain) and the epilogue scales each
// output row by 1 / rms(x) (the scale commutes with the product), so the norm
// needs neither its own launch nor a pass over the activations here.
//
// X1 (17 rows: two row tiles, the second holding only row 16): the first
// tile's activations are resident or streamed as for one tile, and row 16's
// chunk of each wavefront sits in LDS, from which each k-tile's second-tile
// fragment is formed (lanes of rows 17-31 zero).  A 17-row launch then
// issues no more global loads than a 16-row one.
template <typename T, int MT, int NB, int EPI, int XS, bool XROW, int KC, bool X1>
__global__ __launch_bounds__(GEMM_THREADS) void gemm_kernel(const GemmParams p) {
  static_assert(!X1 || MT == 2, "one extra row rides on the second row tile");
  constexpr int E = Ty<T>::E, KT = Ty<T>::KT, ES = Ty<T>::SIZE;
  constexpr int MX = X1 ? 1 : MT;   // row tiles whose activations come from global memory
  constexpr int WAVES = GEMM_WAVES, NT = GEMM_THREADS, U = X1 ? (NB == 2 && XS == 2 ? 2 : 4) : gemm_u<MT, NB>();
  constexpr int NF = MT * NB;
  constexpr int R = MT * 16;
  constexpr bool XRES = KC > 0;
  static_assert(!XRES || (KC % (2 * U)) == 0, "resident chunk: an even number of batches");
  static_assert(NF * 64 <= NT, "one accumulator element per thread");
  constexpr int ROUND = (16 / NF) < WAVES ? (16 / NF) : WAVES;  // wavefronts per LDS round (<= 16 KiB)
  __shared__ f32x4 red[ROUND * NF * 64];
  __shared__ f32x4 tile[NF * 64];
  __shared__ unsigned long long best_row[R];
  // Consumers of an RMSNorm (packed activations into QKV, KV injection,
  // gate/up, the draft head) scale their output rows; the other launches
  // carry no row-scale code.
  constexpr bool RS = !XROW && (EPI == EPI_QKV || EPI == EPI_KVINJ || EPI == EPI_SWIGLU || EPI == EPI_ARGMAX ||
                                EPI == EPI_LOGITS);
  __shared__ float rs_row[RS ? R : 1];
  __shared__ f32x4 rs_stage[RS ? RS_STAGE_FLOATS / 4 : 1];  // tile sums of the block's rows
  // X1: row 16 of every wavefront's k-tiles and planes, four 16-byte chunks each
  __shared__ uint4 x1_lds[X1 ? WAVES * X1_MAX_KTILES * XS * 4 : 1];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n_items = p.m_blocks * p.n_blocks;
  const int my_items = (n_items - int(blockIdx.x) + int(gridDim.x) - 1) / int(gridDim.x);
  // Wavefront w takes the k-tiles w, w + 8, w + 16, ... (its j-th is
  // ktile(j)): the workgroup's loads in flight then cover one contiguous run
  // of the item's weights, and the wavefronts reach the fold together
  // (contiguous per-wavefront chunks arrived several microseconds apart).
  const int per = (p.k_tiles + WAVES - 1) / WAVES;      // k-tiles of the longest wavefront share
  const int nj = p.k_tiles > wave ? (p.k_tiles - wave + WAVES - 1) / WAVES : 0;   // this wavefront's
  const int jlast = nj > 0 ? nj - 1 : 0;
  auto ktile = [&](int j) { return min(wave + WAVES * min(j, jlast), p.k_tiles - 1); };
  const int nbat = XRES ? KC / U : (per + U - 1) / U;   // batches per item, uniform over wavefronts
  const size_t wstride = size_t(p.k_tiles) * 1024;

  if constexpr (EPI == EPI_ARGMAX) {
    if (threadIdx.x < R) best_row[threadIdx.x] = 0;
  }

  auto item_of = [&](int i) { return int(blockIdx.x) + i * int(gridDim.x); };
  // Weight tiles of an item through a buffer resource: the item base and the
  // k-tile offset are uniform (scalar registers); a lane adds only lane * 16.
  // Every k-tile index is clamped into the wavefront's share, so all offsets
  // stay inside the item's NB rows of tiles.  NB == 2 weights use the paired
  // layout (the two row tiles interleave per k-tile), so one k-tile of an
  // item is one contiguous run.
  // live == false: a resource of no bytes, so the loads of a prefetch past
  // the last item return zeros without a memory access (and do not hold up
  // the epilogue's own loads behind them).
  auto w_rsrc = [&](int item, bool live = true) {
    const int nt0 = (item % p.n_blocks) * NB;
    const int seg = nt0 / p.seg_ntiles;
    const char *base = uniform_ptr(p.w_seg[seg] + size_t(nt0 - seg * p.seg_ntiles) * wstride);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), (short)0, live ? int(NB * wstride) : 0,
                                             BUF_DWORD3);
  };
  const int w_lane = lane * 16;
  auto w_off = [&](int kt, int nb) { return NB == 2 ? (kt * 2 + nb) * 1024 : nb * int(wstride) + kt * 1024; };
  // With streamed activations or two row tiles of row-major input, lanes of rows past M load
  // nothing (the packed buffers hold zeros there): the second row tile of a
  // 17-row launch then moves 64 bytes a fragment instead of 1 KiB.  (A
  // resident single tile loads once; the guard would only cost registers.)
  auto x_load = [&](int mtg, int kt, int xp) -> uint4 {
    if constexpr (KC == 0 || (MT > 1 && XROW)) {
      const int row = mtg * 16 + (lane & 15);
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row < p.M) {
        if constexpr (XROW) v = ld16(p.x + (size_t(row) * p.x_ld + kt * KT + (lane >> 4) * E) * ES);
        else v = ld16(p.x + xp * p.x_plane + (size_t(mtg) * p.k_tiles + kt) * 1024 + lane * 16);
      }
      return v;
    } else if constexpr (XROW) {
      const int row = min(mtg * 16 + (lane & 15), p.M - 1);
      return ld16(p.x + (size_t(row) * p.x_ld + kt * KT + (lane >> 4) * E) * ES);
    } else {
      return ld16(p.x + xp * p.x_plane + (size_t(mtg) * p.k_tiles + kt) * 1024 + lane * 16);
    }
  };

  // Accumulator chains: one per k-tile of a batch and activation plane, or
  // one per plane when NB * XS already gives four independent chains.
  constexpr int UC = NB * XS >= 4 ? 1 : 2;
  f32x4 acc[UC][XS][MT][NB];
  auto zero_acc = [&]() {
#pragma unroll
    for (int c = 0; c < UC; ++c)
#pragma unroll
      for (int xp = 0; xp < XS; ++xp)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) acc[c][xp][mt][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  // Chain sum for tile (mt, nb): (c0 + c1) per plane, then hi + lo.
  auto chain_sum = [&](int mt, int nb) -> f32x4 {
    f32x4 r = acc[0][0][mt][nb];
#pragma unroll
    for (int c = 1; c < UC; ++c) r += acc[c][0][mt][nb];
#pragma unroll
    for (int xp = 1; xp < XS; ++xp) {
      f32x4 q = acc[0][xp][mt][nb];
#pragma unroll
      for (int c = 1; c < UC; ++c) q += acc[c][xp][mt][nb];
      r += q;
    }
    return r;
  };
  // chk: zero the weights of k-tiles past the wavefront's chunk (a chunk of
  // exactly the resident length needs no check).
  // kk: the k-tile's index within the wavefront's chunk (X1's LDS row)
  auto mma_tile = [&](int u, int b, const uint4 (&w)[U][NB], const uint4 (&x)[MX][XS], int mblk, int kk,
                      bool chk = true) {
    const bool ok = !chk || b * U + u < nj;
    uint4 x1v[XS];
    if constexpr (X1) {
#pragma unroll
      for (int xp = 0; xp < XS; ++xp) {
        // (k-tiles past the chunk, whose weights are zeroed, read zeros too:
        // that LDS was never written)
        const uint4 r = x1_lds[(wave * X1_MAX_KTILES + kk) * XS * 4 + xp * 4 + (lane >> 4)];
        x1v[xp] = (lane & 15) == 0 && kk < nj ? r : make_uint4(0, 0, 0, 0);
      }
    }
    bool row_ok[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) row_ok[mt] = !XROW || (mblk * MT + mt) * 16 + (lane & 15) < p.M;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint4 wv = ok ? w[u][nb] : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int xp = 0; xp < XS; ++xp) {
          uint4 xv;
          if constexpr (X1) xv = mt == 1 ? x1v[xp] : x[0][xp];
          else xv = x[mt][xp];
          xv = row_ok[mt] ? xv : make_uint4(0, 0, 0, 0);
          acc[u % UC][xp][mt][nb] = mma<T>(acc[u % UC][xp][mt][nb], wv, xv);  // chain = k-tile parity
        }
    }
  };

  int cur_mblk = -1;
  int items_done = 0;
  auto flush_argmax = [&](int mblk) {
    if constexpr (EPI == EPI_ARGMAX) {
      if (threadIdx.x < R) {
        const int m = mblk * R + threadIdx.x;
        if (m < p.M && best_row[threadIdx.x] != 0)
          __hip_atomic_fetch_max(p.keys + size_t(m) * ARGMAX_SLOTS + (blockIdx.x % ARGMAX_SLOTS),
                                 best_row[threadIdx.x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        best_row[threadIdx.x] = 0;
      }
    }
  };
  // Row scales.  Inline (rs_ssq, one row block): the rows' tile sums are
  // loaded before anything else, staged in LDS once the first weight and
  // activation loads are out, and reduced into rs_row while those loads are
  // in flight.  Otherwise (rs_direct) each item's scales are fetched one item
  // ahead into a register and moved to rs_row between the barriers of
  // finish_item, after every reader of the previous values has passed the
  // first barrier.
  float rs_next = 1.f;
  bool rs_first = true;
  f32x4 rs_ld[RS_STAGE_FLOATS / 4 / GEMM_THREADS];
  const int rs_n4 = RS && p.rs_ssq ? min(p.M, R) * p.rs_tiles / 4 : 0;
  auto fetch_rs = [&](int i) {
    if constexpr (RS) {
      if (p.rs_direct && int(threadIdx.x) < R && i < my_items) {
        const int m = (item_of(i) / p.n_blocks) * R + threadIdx.x;
        rs_next = m < p.M ? p.rs_direct[m] : 0.f;
      }
    }
  };
  auto rs_issue = [&]() {
    if constexpr (RS) {
#pragma unroll
      for (int i = 0; i < RS_STAGE_FLOATS / 4 / GEMM_THREADS; ++i) {
        const int c = threadIdx.x + i * GEMM_THREADS;
        if (c < rs_n4) rs_ld[i] = reinterpret_cast<const f32x4 *>(p.rs_ssq)[c];
      }
      fetch_rs(0);
    }
  };
  auto rs_stage_store = [&]() {
    if constexpr (RS) {
      if (p.rs_ssq) {
#pragma unroll
        for (int i = 0; i < RS_STAGE_FLOATS / 4 / GEMM_THREADS; ++i) {
          const int c = threadIdx.x + i * GEMM_THREADS;
          if (c < rs_n4) rs_stage[c] = rs_ld[i];
        }
        lds_barrier();
        const int row = threadIdx.x >> 3;
        if (row < R) {
          const int m = row < p.M ? row : 0;
          const float v = row_rstd8(reinterpret_cast<const float *>(rs_stage) + m * p.rs_tiles, p.rs_tiles,
                                    p.rs_K, p.rs_eps);
          if ((threadIdx.x & 7) == 0) rs_row[row] = v;
        }
      }
    }
  };
  auto place_rs = [&]() {
    if constexpr (RS) {
      if (p.rs_ssq) {
      } else if (p.rs_direct) {
        if (int(threadIdx.x) < R) rs_row[threadIdx.x] = rs_next;
      } else if (rs_first && int(threadIdx.x) < R) {
        rs_row[threadIdx.x] = 1.f;
      }
      rs_first = false;
    }
  };
  // Fold the wavefronts' partial tiles in wavefront order and run the epilogue.
  auto finish_item = [&](int item) {
    const int nblk = item % p.n_blocks, mblk = item / p.n_blocks;
    if constexpr (EPI == EPI_ARGMAX) {
      if (mblk != cur_mblk && cur_mblk >= 0) flush_argmax(cur_mblk);
      cur_mblk = mblk;
    }
    if constexpr (NF <= 2) {
      // All 8 partial tiles fit in LDS at once (<= 16 KiB).
      constexpr int F = NF * 256;  // floats per tile
      float *redf = reinterpret_cast<float *>(red);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) red[(wave * NF + mt * NB + nb) * 64 + lane] = chain_sum(mt, nb);
      lds_barrier();
      place_rs();
      if (int(threadIdx.x) < F) {
        const int f = threadIdx.x;
        float v = redf[f];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) v += redf[w * F + f];
        reinterpret_cast<float *>(tile)[f] = v;
      }
      lds_barrier();
    } else {
      f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
      const int e_own = threadIdx.x;
      for (int r0 = 0; r0 < WAVES; r0 += ROUND) {
        if (wave >= r0 && wave < r0 + ROUND) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) red[((wave - r0) * NF + mt * NB + nb) * 64 + lane] = chain_sum(mt, nb);
        }
        lds_barrier();
        if (e_own < NF * 64) {
          for (int w = 0; w < ROUND; ++w) {
            if (r0 == 0 && w == 0) sum = red[e_own];
            else sum += red[w * NF * 64 + e_own];
          }
        }
        lds_barrier();
      }
      if (e_own < NF * 64) tile[e_own] = sum;
      place_rs();
      lds_barrier();
    }
    gemm_epilogue<T, MT, NB, EPI>(p, tile, RS ? rs_row : nullptr, mblk, nblk, best_row);
    zero_acc();
    fetch_rs(++items_done);
  };

  zero_acc();
  if constexpr (X1) {
    // row 16 of this wavefront's chunk into LDS (only this wavefront reads it)
    const int n = nj * XS * 4;
    for (int c = lane; c < n; c += 64) {
      const int kk = c / (XS * 4), xp = (c / 4) % XS, g = c % 4, kt = wave + WAVES * kk;
      uint4 v;
      if constexpr (XROW) v = ld16(p.x + (size_t(16) * p.x_ld + kt * KT + g * E) * ES);
      else v = ld16(p.x + xp * p.x_plane + (size_t(p.k_tiles) + kt) * 1024 + g * 256);
      x1_lds[(wave * X1_MAX_KTILES + kk) * XS * 4 + xp * 4 + g] = v;
    }
  }
  if constexpr (XRES) {
    constexpr int NBAT = KC / U;
    // A wavefront whose share is exactly KC k-tiles (every share at the
    // drafter's shapes) addresses its weights through a resource based at
    // its first k-tile: every load offset is then a compile-time constant, so
    // no per-k-tile offsets occupy (and spill out of) the scalar registers.
    // Other shares clamp their k-tile indices.
    const bool exact = NB <= 2 && nj == KC;
    auto w_rsrc_chunk = [&](int item, bool live) {
      const int nt0 = (item % p.n_blocks) * NB;
      const int seg = nt0 / p.seg_ntiles;
      const char *base = uniform_ptr(p.w_seg[seg] + size_t(nt0 - seg * p.seg_ntiles) * wstride +
                                     size_t(wave) * NB * 1024);
      return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(base), (short)0,
                                               live ? ((KC - 1) * WAVES + 1) * NB * 1024 : 0, BUF_DWORD3);
    };
    auto body = [&](auto ex) {
    constexpr bool EX = decltype(ex)::value;
    WBatch<U, NB> wb[2];
    auto issue_w = [&](int item, int b, WBatch<U, NB> &f, bool live = true) {
      if constexpr (EX) {
        const auto rs = w_rsrc_chunk(item, live);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            f.w[u][nb] = ld16_buf_stream(rs, w_lane, ((b * U + u) * WAVES * NB + nb) * 1024);
      } else {
        const auto rs = w_rsrc(item, live);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int kt = ktile(b * U + u);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) f.w[u][nb] = ld16_buf_stream(rs, w_lane, w_off(kt, nb));
        }
      }
    };
    rs_issue();
    __builtin_amdgcn_sched_barrier(0);
    issue_w(item_of(0), 0, wb[0]);
    // Activations of this wavefront's chunk, loaded once (one row block) and
    // kept for every item: up to 16 tiles, the first batch's now and each
    // further batch beside the first item's weight batch before it, so the
    // chunk arrives with the first item's weight stream instead of ahead of
    // it.
    uint4 xr[KC][MX][XS];
    auto load_x = [&](int b) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kt = ktile(b * U + u);
#pragma unroll
        for (int mt = 0; mt < MX; ++mt)
#pragma unroll
          for (int xp = 0; xp < XS; ++xp) xr[b * U + u][mt][xp] = x_load(mt, kt, xp);
      }
    };
    // (A 48-tile chunk leaves no registers for the peeled first item: it is
    // loaded whole, up front.)
    constexpr bool PROGRESSIVE = KC <= 16;
    if constexpr (PROGRESSIVE) {
      load_x(0);
    } else {
#pragma unroll
      for (int b = 0; b < NBAT; ++b) load_x(b);
    }
    __builtin_amdgcn_sched_barrier(0);
    rs_stage_store();
    if (PROGRESSIVE && my_items > 0) {
      const int item = item_of(0);
      const int next = item_of(min(1, my_items - 1));
#pragma unroll
      for (int b = 0; b < NBAT; ++b) {
        if (b + 1 < NBAT) {
          issue_w(item, b + 1, wb[(b + 1) & 1]);
          load_x(b + 1);
        } else {
          issue_w(next, 0, wb[0], my_items > 1);
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the next batch's loads ahead of these MFMAs
#pragma unroll
        for (int u = 0; u < U; ++u) mma_tile(u, b, wb[b & 1].w, xr[b * U + u], 0, b * U + u, !EX);
      }
      finish_item(item);
    }
    for (int i = PROGRESSIVE ? 1 : 0; i < my_items; ++i) {
      const int item = item_of(i);
      const int next = item_of(min(i + 1, my_items - 1));
#pragma unroll
      for (int b = 0; b < NBAT; ++b) {
        if (b + 1 < NBAT) issue_w(item, b + 1, wb[(b + 1) & 1]);
        else issue_w(next, 0, wb[0], i + 1 < my_items);
        __builtin_amdgcn_sched_barrier(0);  // keep the next batch's loads ahead of these MFMAs
#pragma unroll
        for (int u = 0; u < U; ++u) mma_tile(u, b, wb[b & 1].w, xr[b * U + u], 0, b * U + u, !EX);
      }
      finish_item(item);
    }
    };
    if (exact) body(std::integral_constant<bool, true>{});
    else body(std::integral_constant<bool, false>{});
  } else {
    // Activations stream with the weights; two batches in flight.
    XWBatch<U, MX, NB, XS> fa, fb;
    const int T_steps = my_items * nbat;
    const int t_last = T_steps - 1;
    auto issue = [&](int t, XWBatch<U, MX, NB, XS> &f) {
      const int item = item_of(t / nbat);
      const int b = t % nbat;
      const int mblk = item / p.n_blocks;
      const auto rs = w_rsrc(item);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kt = ktile(b * U + u);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) f.w[u][nb] = ld16_buf_stream(rs, w_lane, w_off(kt, nb));
#pragma unroll
        for (int mt = 0; mt < MX; ++mt)
#pragma unroll
          for (int xp = 0; xp < XS; ++xp) f.x[u][mt][xp] = x_load(mblk * MT + mt, kt, xp);
      }
    };
    auto compute = [&](int t, const XWBatch<U, MX, NB, XS> &f) {
      const int b = t % nbat;
      const int mblk = item_of(t / nbat) / p.n_blocks;
#pragma unroll
      for (int u = 0; u < U; ++u) mma_tile(u, b, f.w, f.x[u], mblk, min(b * U + u, jlast));
    };
    rs_issue();
    __builtin_amdgcn_sched_barrier(0);
    issue(0, fa);
    __builtin_amdgcn_sched_barrier(0);
    rs_stage_store();
    for (int t = 0; t < T_steps; t += 2) {
      issue(min(t + 1, t_last), fb);
      __builtin_amdgcn_sched_barrier(0);
      compute(t, fa);
      if (t % nbat == nbat - 1) finish_item(item_of(t / nbat));
      issue(min(t + 2, t_last), fa);
      __builtin_amdgcn_sched_barrier(0);
      if (t + 1 < T_steps) {
        compute(t + 1, fb);
        if ((t + 1) % nbat == nbat - 1) finish_item(item_of((t + 1) / nbat));
      }
    }
  }
  if constexpr (EPI == EPI_ARGMAX) {
    lds_barrier();
    if (cur_mblk >= 0) flush_argmax(cur_mblk);
  }
  if constexpr (EPI == EPI_ARGMAX || EPI == EPI_KVINJ) {
    if (p.arrive) {
      __shared__ int flag;
      __shared__ int toks[FUSED_FINISH_ROWS];
      if (last_arriver(p.arrive, &flag)) {
        if constexpr (EPI == EPI_ARGMAX) {
          fused_argmax_finish(p.fin, p.M, toks);
        } else {
          // commit: ctx_len[s] += n_s unless the injection skipped sequence s
          for (int s = threadIdx.x; s < p.batch; s += blockDim.x) {
            const int ns = p.cu_new[s + 1] - p.cu_new[s];
            if (p.ctx_len_w[s] + ns <= p.capacity) p.ctx_len_w[s] += ns;
          }
        }
        if (threadIdx.x == 0) __hip_atomic_store(p.arrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// One workgroup per sequence: fold the argmax slots of its rows, clear them
// for the next launch, write the token ids and, for verification, the
// accepted length and the fallback token.
__global__ __launch_bounds__(256) void argmax_finish_kernel(const ArgmaxFinishParams p) {
  __shared__ int toks[32];
  const int s = blockIdx.x;
  const int R = p.rows_per_seq;
  for (int r = threadIdx.x; r < R; r += blockDim.x) {
    const int m = s * R + r;
    unsigned long long best = 0;
    unsigned long long *k = p.keys + size_t(m) * ARGMAX_SLOTS;
    for (int i = 0; i < ARGMAX_SLOTS; ++i) {
      const unsigned long long v = k[i];
      best = v > best ? v : best;
      k[i] = 0;
    }
    const int tok = key_index(best);
    p.tok_out[m] = tok;
    toks[r] = tok;
  }
  __syncthreads();
  if (p.verify && threadIdx.x == 0) {
    const int B = p.block;
    int L = B;
    for (int j = 0; j < B; ++j) {
      if (p.draft_in[s * B + j] != toks[j]) { L = j; break; }
    }
    p.accept_len[s] = L;
    p.bonus[s] = toks[L];
  }
}

template <typename T, int MT, int NB, int EPI, int XS, bool XROW, int KC, bool X1 = false>
static hipError_t launch_one(const GemmParams &p, hipStream_t s) {
  const int items = p.m_blocks * p.n_blocks;
  const dim3 grid(items < p.grid_cap ? items : p.grid_cap);
  hipLaunchKernelGGL((gemm_kernel<T, MT, NB, EPI, XS, XROW, KC, X1>), grid, dim3(GEMM_THREADS), 0, s, p);
  return hipGetLastError();
}

// Resident activations when gemm_resident_ok holds; the chunk register array
// is sized 4 (batches of two only), 8 or 16 tiles (32 or 48 for one row tile and
// plane, NB == 1).
template <typename T, int MT, int NB, int EPI, int XS, bool XROW>
static hipError_t launch_kc(const GemmParams &p, hipStream_t s) {
  const int per = (p.k_tiles + GEMM_WAVES - 1) / GEMM_WAVES;
  if constexpr (MT * XS <= 2) {
    if (gemm_resident_ok(p.m_blocks, MT, XS, p.k_tiles)) {
      if constexpr (gemm_u<MT, NB>() == 2) {
        if (per <= 4) return launch_one<T, MT, NB, EPI, XS, XROW, 4>(p, s);
      }
      if (per <= 8) return launch_one<T, MT, NB, EPI, XS, XROW, 8>(p, s);
      if (per <= 16) return launch_one<T, MT, NB, EPI, XS, XROW, 16>(p, s);
      if constexpr (MT * XS == 1 && NB == 1) {
        if (per <= 32) return launch_one<T, MT, NB, EPI, XS, XROW, 32>(p, s);
        return launch_one<T, MT, NB, EPI, XS, XROW, 48>(p, s);
      }
    }
  }
  return launch_one<T, MT, NB, EPI, XS, XROW, 0>(p, s);
}

// 17 rows (a 16-slot block's verify pass at batch 1): the first row tile as
// one tile, row 16 through LDS; the first tile's activations resident when
// its chunk is at most 16 tiles, else streamed.
template <typename T, int NB, int EPI, int XS, bool XROW>
static hipError_t launch_x1(const GemmParams &p, hipStream_t s) {
  const int per = (p.k_tiles + GEMM_WAVES - 1) / GEMM_WAVES;
  if constexpr (XS <= 2) {
    if (gemm_resident_ok(p.m_blocks, 1, XS, p.k_tiles)) {
      if (per <= 8) return launch_one<T, 2, NB, EPI, XS, XROW, 8, true>(p, s);
      if (per <= 16) return launch_one<T, 2, NB, EPI, XS, XROW, 16, true>(p, s);
    }
  }
  return launch_one<T, 2, NB, EPI, XS, XROW, 0, true>(p, s);
}

template <typename T, int EPI, int NB, int XS, bool XROW>
static hipError_t launch_xs(const GemmParams &p, hipStream_t s) {
  const int per = (p.k_tiles + GEMM_WAVES - 1) / GEMM_WAVES;
  switch (p.MT) {
    case 1: return launch_kc<T, 1, NB, EPI, XS, XROW>(p, s);
    case 2:
      if (p.M == 17 && p.m_blocks == 1 && per <= X1_MAX_KTILES) return launch_x1<T, NB, EPI, XS, XROW>(p, s);
      return launch_kc<T, 2, NB, EPI, XS, XROW>(p, s);
    default: return hipErrorInvalidValue;   // more than 32 rows run tiled
  }
}

// Activation planes: fp32 storage always has one; bf16 activations that the
// step produces itself carry two (hi + lo); external row-major inputs (target
// features, target hidden states) one.
template <typename T, int EPI, int NB>
static hipError_t launch_mt(const GemmParams &p, hipStream_t s) {
  if (p.x_ld > 0) return p.xs == 1 ? launch_xs<T, EPI, NB, 1, true>(p, s) : hipErrorInvalidValue;
  if constexpr (Ty<T>::SIZE == 2) {
    if (p.xs == 2) return launch_xs<T, EPI, NB, 2, false>(p, s);
  }
  return p.xs == 1 ? launch_xs<T, EPI, NB, 1, false>(p, s) : hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_t(int epi, const GemmParams &p, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: return p.NB == 1 ? launch_mt<T, EPI_STORE, 1>(p, s) : hipErrorInvalidValue;
    case EPI_RESID: return p.NB == 1 ? launch_mt<T, EPI_RESID, 1>(p, s) : hipErrorInvalidValue;
    case EPI_QKV: return p.NB == 1 ? launch_mt<T, EPI_QKV, 1>(p, s) : hipErrorInvalidValue;
    case EPI_KVINJ: return p.NB == 1 ? launch_mt<T, EPI_KVINJ, 1>(p, s) : hipErrorInvalidValue;
    case EPI_SWIGLU: return p.NB == 2 ? launch_mt<T, EPI_SWIGLU, 2>(p, s) : hipErrorInvalidValue;
    case EPI_ARGMAX: return p.NB == 2 ? launch_mt<T, EPI_ARGMAX, 2>(p, s) : hipErrorInvalidValue;
    case EPI_LOGITS: return p.NB == 2 ? launch_mt<T, EPI_LOGITS, 2>(p, s) : hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm(int dtype, int epi, const GemmParams &p, hipStream_t s) {
  if (p.tiled) return launch_gemm_tiled(dtype, epi, p, s);
  return dtype == DFLASH_BF16 ? launch_t<bf16_t>(epi, p, s) : launch_t<float>(epi, p, s);
}

hipError_t launch_argmax_finish(const ArgmaxFinishParams &p, int batch, hipStream_t s) {
  hipLaunchKernelGGL(argmax_finish_kernel, dim3(batch), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace dflash
