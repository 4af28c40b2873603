// Y = X W^T on MFMA for launches with many rows (draft and verify GEMMs of
// more than 17 rows, injections of more than 32: the batched draft step and
// its heads, large injections).
//
// A workgroup owns a TM x TN tile of 16 x 16 output fragments (128 tokens x
// 256 features, or 64 x 128 when the large tiles would leave compute units
// idle) and the whole K range; its 8 wavefronts form a 2 x 4 grid of
// sub-tiles, each accumulating (TM / 2) x (TN / 4) MFMA fragments over all of
// K.  Per 32-column k-tile the tile's activation fragments (TM row tiles, one
// or two planes) and weight fragments (TN row tiles) are copied straight from
// global memory into an LDS ring of as many stages as fit 144 KiB (global_load_lds_dwordx4, one
// 1 KiB fragment per wavefront instruction, the same number for every
// wavefront so the wait before a stage is an immediate); every wavefront then
// reads its fragments from LDS, so each fragment fetched from L2 feeds
// several MFMAs.  Tiles are spread over the 8 XCDs so that an XCD's
// workgroups take every 8th feature block with all of its token blocks: the
// weight fragments they share meet in that XCD's L2.  Workgroups walk their
// tiles with the k-tile pipeline running across tile boundaries.  Epilogues
// work on the accumulator registers directly: lane (c, g) of a fragment
// holds token c and features 4g .. 4g + 3.
#include "common.hpp"
#include "kernels.hpp"
#include "gemm_util.hpp"

namespace dflash {

constexpr int TL_XCDS = 8;   // workgroups are dispatched round-robin over 8 XCDs

// S: stages of the LDS ring; S - 1 of them are in flight while one is consumed.
// WGM x WGN wavefronts; each owns (TM / WGM) x (TN / WGN) fragments.
template <typename T, int EPI, int XS, bool XROW, int TM, int TN, int S, int WGM, int WGN>
__global__ __launch_bounds__(WGM * WGN * 64) void gemm_tiled_kernel(const GemmParams p) {
  constexpr int TL_WAVES = WGM * WGN;
  constexpr int TL_STAGES = S;
  constexpr int E = Ty<T>::E, KT = Ty<T>::KT, ES = Ty<T>::SIZE;
  constexpr int TL_MT = TM, TL_NT = TN;
  constexpr int TL_WM = TM / WGM, TL_WN = TN / WGN;   // fragments per wavefront
  static_assert(TL_WM * WGM == TM && TL_WN * WGN == TN, "wave grid divides the tile");
  static_assert(TM * 16 <= TL_WAVES * 64, "one thread per token row of the tile");
  // two-tile items (gate/up pairs, the heads) use the paired weight layout
  constexpr bool PAIRED = EPI == EPI_SWIGLU || EPI == EPI_ARGMAX || EPI == EPI_LOGITS;
  constexpr bool RS = !XROW && (EPI == EPI_QKV || EPI == EPI_KVINJ || EPI == EPI_SWIGLU || EPI == EPI_ARGMAX ||
                                EPI == EPI_LOGITS);
  constexpr int XT = TL_MT * XS;                              // activation fragments per stage
  constexpr int ST = XT + TL_NT;                              // fragments per stage
  constexpr int LPW = (ST + TL_WAVES - 1) / TL_WAVES;         // loads per wavefront per stage
  constexpr int SP = LPW * TL_WAVES;                          // stage slots (the last SP - ST unused)
  static_assert(TL_WN % 2 == 0 || !PAIRED, "pairs stay inside a wavefront");
  __shared__ uint4 ring[TL_STAGES * SP * 64];
  __shared__ unsigned long long best_row[TL_MT * 16];
  __shared__ int flag;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int wm = wave / WGN, wn = wave % WGN;
  const int c = lane & 15, g = lane >> 4;
  const int K = p.k_tiles;
  // Work units: an item (feature block, token block) or, with ksplit > 1,
  // one of ksplit parts of its k-tile range.  XCD-aware order (the grid is a
  // multiple of 8): XCD x takes feature blocks x, x + 8, ...; its workgroups
  // walk those blocks' units with the part fastest, then the token block.
  const int xcd = int(blockIdx.x) % TL_XCDS, r = int(blockIdx.x) / TL_XCDS;
  const int per_xcd = int(gridDim.x) / TL_XCDS;
  const int ks = p.ksplit;
  const int nb_x = (p.n_blocks - xcd + TL_XCDS - 1) / TL_XCDS;
  const int units_x = nb_x * p.m_blocks * ks;
  const int my_items = (units_x - r + per_xcd - 1) / per_xcd;
  // unit index (item * ks + part) of this workgroup's i-th unit
  auto item_of = [&](int i) {
    const int li = r + i * per_xcd;
    const int per_nb = p.m_blocks * ks;
    return (xcd + TL_XCDS * (li / per_nb)) * per_nb + li % per_nb;
  };
  auto k_begin = [&](int unit) { return (unit % ks) * K / ks; };
  auto k_end = [&](int unit) { return (unit % ks + 1) * K / ks; };
  int steps = 0;
  for (int i = 0; i < my_items; ++i) steps += k_end(item_of(i)) - k_begin(item_of(i));

  // Issue side: the next stage to load (item, k-tile, ring slot), and per
  // load of this wavefront a wave-uniform base at k-tile 0 of the item, the
  // lane's byte offset from it and the bytes per k-tile (set once per item,
  // so a stage costs only scalar arithmetic).
  int is_i = 0, is_kt = 0, is_slot = 0, issued = 0;
  const char *sb[LPW];
  uint32_t vo[LPW];
  int fstep[LPW];
  const uint32_t lane16 = uint32_t(lane) * 16u;
  int is_kend = 0;
  auto set_item = [&](int i) {
    const int unit = item_of(i), item = unit / ks;
    const int nblk = item / p.m_blocks, mblk = item % p.m_blocks;
    is_kt = k_begin(unit);
    is_kend = k_end(unit);
#pragma unroll
    for (int l = 0; l < LPW; ++l) {
      const int j = wave + l * TL_WAVES;
      const char *base;
      vo[l] = lane16;
      if (j >= ST) {
        base = p.w_seg[0];   // padding slot: any valid fragment
        fstep[l] = 0;
      } else if (j < XT) {
        const int mt = j / XS, xp = j % XS;
        if constexpr (XROW) {
          // rows past M repeat row M - 1 (their results are never stored)
          const int r0 = (mblk * TL_MT + mt) * 16, rb = min(r0, p.M - 1), row = min(r0 + c, p.M - 1);
          base = p.x + size_t(rb) * p.x_ld * ES;
          vo[l] = uint32_t(((row - rb) * p.x_ld + g * E) * ES);
          fstep[l] = KT * ES;
        } else {
          const int mg = min(mblk * TL_MT + mt, p.x_mtiles - 1);
          base = p.x + size_t(xp) * p.x_plane + size_t(mg) * K * 1024;
          fstep[l] = 1024;
        }
      } else {
        const int nt = min(nblk * TL_NT + (j - XT), p.n_tiles - 1);
        const int seg = nt / p.seg_ntiles, loc = nt - seg * p.seg_ntiles;
        if constexpr (PAIRED) {
          base = p.w_seg[seg] + (size_t(loc >> 1) * K * 2 + (loc & 1)) * 1024;
          fstep[l] = 2048;
        } else {
          base = p.w_seg[seg] + size_t(loc) * K * 1024;
          fstep[l] = 1024;
        }
      }
      sb[l] = uniform_ptr(base);
    }
  };
  auto issue_next = [&]() {
    uint4 *slot = ring + is_slot * SP * 64;
#pragma unroll
    for (int l = 0; l < LPW; ++l)
      load_lds16_s(sb[l] + size_t(is_kt) * fstep[l], vo[l], slot + (wave + l * TL_WAVES) * 64);
    ++issued;
    is_slot = is_slot + 1 == TL_STAGES ? 0 : is_slot + 1;
    if (++is_kt == is_kend && ++is_i < my_items) set_item(is_i);
  };

  f32x4 acc[TL_WM][TL_WN];
  auto zero = [&]() {
#pragma unroll
    for (int a = 0; a < TL_WM; ++a)
#pragma unroll
      for (int b = 0; b < TL_WN; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  // A wavefront's fragments of one stage, double-buffered in registers: the
  // LDS reads of stage t + 1 are in flight while the MFMAs of stage t run.
  struct Frags {
    uint4 x[TL_WM][XS];
    uint4 w[TL_WN];
  };
  auto read_frags = [&](int slot_idx, Frags &f) {
    const uint4 *slot = ring + slot_idx * SP * 64;
#pragma unroll
    for (int a = 0; a < TL_WM; ++a)
#pragma unroll
      for (int xp = 0; xp < XS; ++xp) f.x[a][xp] = slot[((wm * TL_WM + a) * XS + xp) * 64 + lane];
#pragma unroll
    for (int b = 0; b < TL_WN; ++b) f.w[b] = slot[(XT + wn * TL_WN + b) * 64 + lane];
  };
  auto mfma_frags = [&](const Frags &f) {
#pragma unroll
    for (int b = 0; b < TL_WN; ++b)
#pragma unroll
      for (int a = 0; a < TL_WM; ++a)
#pragma unroll
        for (int xp = 0; xp < XS; ++xp) acc[a][b] = mma<T>(acc[a][b], f.w[b], f.x[a][xp]);
  };

  int cur_mblk = -1;
  auto flush_argmax = [&](int mblk) {
    if constexpr (EPI == EPI_ARGMAX) {
      __syncthreads();
      if (int(threadIdx.x) < TL_MT * 16) {
        const int m = mblk * TL_MT * 16 + threadIdx.x;
        if (m < p.M && best_row[threadIdx.x] != 0)
          __hip_atomic_fetch_max(p.keys + size_t(m) * ARGMAX_SLOTS + (blockIdx.x % ARGMAX_SLOTS), best_row[threadIdx.x],
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        best_row[threadIdx.x] = 0;
      }
      __syncthreads();
    }
  };

  auto epilogue = [&](int item) {
    const int nblk = item / p.m_blocks, mblk = item % p.m_blocks;
    if constexpr (EPI == EPI_ARGMAX) {
      if (mblk != cur_mblk) {
        if (cur_mblk >= 0) flush_argmax(cur_mblk);
        cur_mblk = mblk;
      }
    }
#pragma unroll
    for (int a = 0; a < TL_WM; ++a) {
      const int ml = (wm * TL_WM + a) * 16 + c;   // token within the tile
      const int m = mblk * TL_MT * 16 + ml;
      const bool mok = m < p.M;
      float rs = 1.f;
      if constexpr (RS) {
        if (p.rs_direct) rs = mok ? p.rs_direct[m] : 0.f;
      }
      if constexpr (EPI == EPI_ARGMAX) {
        unsigned long long k = 0;
#pragma unroll
        for (int b = 0; b < TL_WN; ++b) {
          const int n0 = (nblk * TL_NT + wn * TL_WN + b) * 16 + 4 * g;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (n0 + i < p.vocab) {
              const unsigned long long kk = argmax_key(acc[a][b][i] * rs, n0 + i);
              k = kk > k ? kk : k;
            }
          }
        }
        unsigned long long o = __shfl_xor(k, 16, 64);
        k = o > k ? o : k;
        o = __shfl_xor(k, 32, 64);
        k = o > k ? o : k;
        if (g == 0 && mok) __hip_atomic_fetch_max(best_row + ml, k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      } else if constexpr (EPI == EPI_LOGITS) {
#pragma unroll
        for (int b = 0; b < TL_WN; ++b) {
          const int n0 = (nblk * TL_NT + wn * TL_WN + b) * 16 + 4 * g;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (mok && n0 + i < p.vocab) p.out_f32[size_t(m) * p.ld_out + n0 + i] = acc[a][b][i] * rs;
        }
      } else if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int b = 0; b < TL_WN; b += 2) {
          const int pair = (nblk * TL_NT + wn * TL_WN + b) >> 1;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int col = pair * 16 + 4 * g + i;
            float out = 0.f;
            if (mok) {
              const float gt = acc[a][b][i] * rs, up = acc[a][b + 1][i] * rs;
              out = gt / (1.0f + __expf(-gt)) * up;
            }
            if (m < p.x_mtiles * 16 && pair < p.n_tiles / 2)  // padded rows get zeros
              store_split<T>(p.out_packed + packed_offset<T>(m, col, p.out_kt), p.out_plane, p.out_planes, out);
          }
        }
      } else {
#pragma unroll
        for (int b = 0; b < TL_WN; ++b) {
          const int ntg = nblk * TL_NT + wn * TL_WN + b;
          const int n0 = ntg * 16 + 4 * g;
          const bool nok = ntg < p.n_tiles;
          f32x4 v = acc[a][b] * rs;
          if constexpr (EPI == EPI_STORE || EPI == EPI_RESID) {
            const size_t o = size_t(m) * p.ld_out + n0;
            if (mok && nok) {
              if constexpr (EPI == EPI_RESID) v += *reinterpret_cast<const f32x4 *>(p.resid + o);
              *reinterpret_cast<f32x4 *>(p.out_f32 + o) = v;
              if (p.aux_out) {
#pragma unroll
                for (int i = 0; i < 4; ++i) store_elem<T>(p.aux_out + (size_t(m) * p.aux_ld + n0 + i) * ES, v[i]);
              }
            } else {
              v = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            if (p.nx_packed && nok && m < p.nx_rows) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float y = v[i] * to_f32<T>(reinterpret_cast<const T *>(p.nx_gain)[n0 + i]);
                store_split<T>(p.nx_packed + packed_offset<T>(m, n0 + i, p.nx_kt), p.nx_plane, p.nx_planes, y);
              }
            }
            if (p.ssq_out) {
              // the balanced tree of tile_ssq16: in-lane pairs, then g ^ 1, g ^ 2
              float s = (__fmul_rn(v[0], v[0]) + __fmul_rn(v[1], v[1])) + (__fmul_rn(v[2], v[2]) + __fmul_rn(v[3], v[3]));
              s += __shfl_xor(s, 16, 64);
              s += __shfl_xor(s, 32, 64);
              if (g == 0 && mok && nok) p.ssq_out[size_t(m) * p.ssq_ld + ntg] = s;
            }
          } else if constexpr (EPI == EPI_QKV) {
            const int d = p.head_dim, nqd = p.n_q * d, nkd = p.n_kv * d;
            const int dt_count = d / KT;
            const int sq = m / p.block, j = m % p.block;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float partner = __shfl_xor(v[i], 32, 64);  // feature n ^ 8: lane g ^ 2
              const int n = n0 + i;
              if (!(mok && nok)) continue;
              float x = v[i];
              if (n < nqd + nkd) {
                const int dd = rot_channel(n % d, d);
                x = rope_apply(x, partner, dd, d, p.ctx_len[sq] + (p.row_pos ? p.row_pos[m] : j), p);
                if (n < nqd) {
                  char *base = p.qbuf + (size_t(sq) * p.n_q + n / d) * p.q_tiles * dt_count * 1024;
                  store_split<T>(base + packed_offset<T>(j, dd, dt_count), p.q_plane, p.q_planes, x);
                } else {
                  char *base = p.kblk + (size_t(sq) * p.n_kv + (n - nqd) / d) * size_t(KT) * d * ES;
                  store_elem<T>(base + kcache_offset<T>(j, dd, d), x);
                  if (p.qkv_to_cache) qkv_cache_store<T>(p, true, sq, (n - nqd) / d, p.ctx_len[sq] + j, dd, x);
                }
              } else {
                const int cc = n - nqd - nkd;
                char *base = p.vblk + (size_t(sq) * p.n_kv + cc / d) * size_t(KT) * d * ES;
                store_elem<T>(base + vcache_offset<T>(j, cc % d, d), x);
                if (p.qkv_to_cache) qkv_cache_store<T>(p, false, sq, cc / d, p.ctx_len[sq] + j, cc % d, x);
              }
            }
          } else if constexpr (EPI == EPI_KVINJ) {
            const int d = p.head_dim, nkd = p.n_kv * d, segn = 2 * nkd;
            const size_t region = size_t(p.capacity) * d * ES;
            int sq = 0, start = 0, ns = 0, C = 0;
            if (mok) {
              int lo = 0, hi = p.batch;  // cu_new[lo] <= m < cu_new[lo + 1]
              while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (p.cu_new[mid] <= m) lo = mid; else hi = mid;
              }
              sq = lo;
              start = p.cu_new[sq];
              ns = p.cu_new[sq + 1] - start;
              C = p.ctx_len[sq];
            }
            const bool fits = C + ns <= p.capacity;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float partner = __shfl_xor(v[i], 32, 64);
              const int n = n0 + i;
              if (!(mok && nok)) continue;
              if (!fits) {
                if (m == start && n == 0) atomicOr(p.status, DFLASH_STATUS_CAPACITY);
                continue;
              }
              const int pos = C + (m - start);
              const int layer = p.layer0 + n / segn, cc = n % segn;
              if (cc < nkd) {
                const int dd = rot_channel(cc % d, d);
                const float r = rope_apply(v[i], partner, dd, d, pos, p);
                char *base = p.kcache + ((size_t(layer) * p.max_batch + sq) * p.n_kv + cc / d) * region;
                store_elem<T>(base + kcache_offset<T>(pos, dd, d), r);
              } else {
                const int c2 = cc - nkd;
                char *base = p.vcache + ((size_t(layer) * p.max_batch + sq) * p.n_kv + c2 / d) * region;
                store_elem<T>(base + vcache_offset<T>(pos, c2 % d, d), v[i]);
              }
            }
          }
        }
      }
    }
    zero();
  };

  if constexpr (EPI == EPI_ARGMAX) {
    if (int(threadIdx.x) < TL_MT * 16) best_row[threadIdx.x] = 0;
    __syncthreads();
  }
  zero();
  if (my_items > 0) set_item(0);
#pragma unroll
  for (int t = 0; t < S - 1; ++t)
    if (issued < steps) issue_next();
  // Consumer side.  Before reading stage t + 1: its loads have landed for
  // this wavefront (vmcnt; with all S - 1 later stages issued S - 2 of them
  // may still be out, otherwise wait for all), the barrier makes that true
  // for every wavefront and frees the slot read one step earlier (stage t's,
  // whose fragments are in registers), which the next stage then reuses.
  // Stage loads retire in order among themselves; after an epilogue's stores
  // and atomics the count no longer says which, so the next wait is for all.
  bool after_epi = false;
  auto wait_stage = [&](int t) {
    if (!after_epi && issued == t + S - 1) wait_vmcnt<(S - 2) * LPW>();
    else wait_vmcnt<0>();
    after_epi = false;
  };
  int rd_slot = 0, t = 0;
  Frags fa, fb2;
  auto step = [&](const Frags &cur, Frags &nxt) {
    if (t + 1 < steps) {
      wait_stage(t + 1);
      lds_barrier();
      if (issued < steps) issue_next();
      rd_slot = rd_slot + 1 == TL_STAGES ? 0 : rd_slot + 1;
      read_frags(rd_slot, nxt);
    }
    mfma_frags(cur);
    ++t;
  };
  if (steps > 0) {
    wait_stage(0);
    lds_barrier();
    if (issued < steps) issue_next();
    read_frags(0, fa);
  }
  // The parts of a split item meet in the workspace: each stores its partial
  // tile (agent-coherent stores, one f32x4 slot per lane and fragment),
  // waits for them and counts itself in; the last to arrive sums the parts
  // in part order from the workspace, so the result does not depend on
  // which part finished last, resets the count and runs the epilogue.
  auto split_last = [&](int unit) -> bool {
    const int item = unit / ks;
    // Fragment (a, b) of a wavefront is 256 floats; element i of every lane
    // is a run of 64 consecutive floats, so each coherent store and load
    // instruction moves one contiguous 256-byte run.
    auto slot = [&](int u, int a, int b) {
      return p.part_ws + ((size_t(u) * TL_WAVES + wave) * (TL_WM * TL_WN) + a * TL_WN + b) * 256 + lane;
    };
#pragma unroll
    for (int a = 0; a < TL_WM; ++a)
#pragma unroll
      for (int b = 0; b < TL_WN; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          __hip_atomic_store(slot(unit, a, b) + i * 64, acc[a][b][i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!last_arriver_of(p.part_cnt + item, unsigned(ks), &flag)) {
      zero();
      return false;
    }
    if (threadIdx.x == 0) __hip_atomic_store(p.part_cnt + item, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int j = 0; j < ks; ++j) {
#pragma unroll
      for (int a = 0; a < TL_WM; ++a)
#pragma unroll
        for (int b = 0; b < TL_WN; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = __hip_atomic_load(slot(item * ks + j, a, b) + i * 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            acc[a][b][i] = j == 0 ? v : acc[a][b][i] + v;
          }
    }
    return true;
  };

  // Two k-tiles per trip so the register buffers alternate without copies;
  // one epilogue per item, after its last k-tile.
  for (int it = 0; it < my_items; ++it) {
    const int unit = item_of(it), nk = k_end(unit) - k_begin(unit);
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      step(fa, fb2);
      step(fb2, fa);
    }
    if (kt < nk) {   // odd k-tile count: the next unit starts from fb2
      step(fa, fb2);
      fa = fb2;
    }
    if (ks == 1 || split_last(unit)) epilogue(unit / ks);
    after_epi = true;
  }
  if constexpr (EPI == EPI_ARGMAX) {
    if (cur_mblk >= 0) flush_argmax(cur_mblk);
  }
  if constexpr (EPI == EPI_KVINJ) {
    if (p.arrive && last_arriver(p.arrive, &flag)) {
      for (int s = threadIdx.x; s < p.batch; s += blockDim.x) {
        const int ns = p.cu_new[s + 1] - p.cu_new[s];
        if (p.ctx_len_w[s] + ns <= p.capacity) p.ctx_len_w[s] += ns;
      }
      if (threadIdx.x == 0) __hip_atomic_store(p.arrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Stages that fit a 144 KiB ring (the LDS holds 160 KiB per workgroup).
template <int TM, int TN, int XS, int WAVES>
constexpr int tl_stages() {
  constexpr int slots = (TM * XS + TN + WAVES - 1) / WAVES * WAVES;
  return 144 / slots;
}

template <typename T, int EPI, int XS, bool XROW, int TM, int TN, int WGM, int WGN>
static void launch_tiled_shape(const GemmParams &p, int grid, hipStream_t s) {
  constexpr int S = tl_stages<TM, TN, XS, WGM * WGN>();
  hipLaunchKernelGGL((gemm_tiled_kernel<T, EPI, XS, XROW, TM, TN, S, WGM, WGN>), dim3(grid), dim3(WGM * WGN * 64), 0, s, p);
}

// Tile choice, 8 wavefronts in a 2 x 4 grid:
//   heads (argmax): TM x 16 fragments with TM even, at most 12: one token
//     block covering every row when it fits (each weight byte read once),
//     else 8 or 12, whichever pads the rows less; the TM = 8 head with one
//     activation plane is 24 fragments wide;
//   others: 8 x 16 (128 tokens x 256 features) when those items fill at
//     least 3/4 of the compute units, else 4 x 8 (64 x 128), with split-K
//     when the items still leave half the units idle.
template <typename T, int EPI, int XS, bool XROW>
static hipError_t launch_tiled_one(const GemmParams &p0, hipStream_t s) {
  GemmParams p = p0;
  const int cu = p.grid_cap;
  auto blocks = [](int n, int b) { return (n + b - 1) / b; };
  const int mt = blocks(p.M, 16);
  constexpr bool HEAD = EPI == EPI_ARGMAX || EPI == EPI_LOGITS;   // vocabulary-wide heads
  if (HEAD) {
    // at least 4 fragments: 2 (17-32 rows) would leave half the wave grid
    // without a row tile
    if (mt <= 12) p.tile_m = mt <= 4 ? 4 : (mt + 1) & ~1;
    else p.tile_m = blocks(mt, 12) * 12 < blocks(mt, 8) * 8 ? 12 : 8;
    // the 128-row head tile is 384 features wide (one plane of activations
    // leaves the registers for it; at 10 and 12 fragments that width spills):
    // each staged weight fragment feeds more MFMAs
    p.n_blocks = blocks(p.n_tiles, (XS == 1 && p.tile_m == 8) ? 24 : 16);
  } else {
    // (the rotary QKV epilogue keeps the 64 x 128 tile: at 128 x 256 its
    // partner exchange does not fit the registers)
    const bool big = EPI != EPI_QKV && blocks(p.M, 128) * blocks(p.n_tiles, 16) * 4 >= 3 * cu;
    p.tile_m = big ? 8 : 4;
    p.n_blocks = big ? blocks(p.n_tiles, 16) : blocks(p.n_tiles, 8);
  }
  p.m_blocks = blocks(p.M, 16 * p.tile_m);
  const int items = p.m_blocks * p.n_blocks;
  // Too few items for the compute units: split each item's k-tiles into
  // parts of at least 16.
  p.ksplit = 1;
  if (!HEAD && p.part_ws && p.part_cnt && 2 * items <= cu) {
    const int cap = cu < MAX_SPLIT_UNITS ? cu : MAX_SPLIT_UNITS;
    int ks = cap / items;
    if (ks > p.k_tiles / 16) ks = p.k_tiles / 16;
    p.ksplit = ks > 1 ? ks : 1;
  }
  // grid: a multiple of the 8 XCDs, at most one workgroup per compute unit
  const int units = items * p.ksplit;
  int grid = units < cu ? units : cu;
  grid = grid < TL_XCDS ? TL_XCDS : grid - grid % TL_XCDS;
  if constexpr (HEAD && XS == 1) {
    switch (p.tile_m) {
      case 4: launch_tiled_shape<T, EPI, XS, XROW, 4, 16, 2, 4>(p, grid, s); break;
      case 6: launch_tiled_shape<T, EPI, XS, XROW, 6, 16, 2, 4>(p, grid, s); break;
      case 8: launch_tiled_shape<T, EPI, XS, XROW, 8, 24, 2, 4>(p, grid, s); break;
      case 10: launch_tiled_shape<T, EPI, XS, XROW, 10, 16, 2, 4>(p, grid, s); break;
      case 12: launch_tiled_shape<T, EPI, XS, XROW, 12, 16, 2, 4>(p, grid, s); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    if (HEAD && p.tile_m != 8) return hipErrorInvalidValue;
    if constexpr (EPI == EPI_QKV) launch_tiled_shape<T, EPI, XS, XROW, 4, 8, 2, 4>(p, grid, s);
    else if (p.tile_m == 8) launch_tiled_shape<T, EPI, XS, XROW, 8, 16, 2, 4>(p, grid, s);
    else launch_tiled_shape<T, EPI, XS, XROW, 4, 8, 2, 4>(p, grid, s);
  }
  return hipGetLastError();
}

template <typename T, int EPI>
static hipError_t launch_tiled_x(const GemmParams &p, hipStream_t s) {
  if (p.x_ld > 0) return p.xs == 1 ? launch_tiled_one<T, EPI, 1, true>(p, s) : hipErrorInvalidValue;
  if constexpr (Ty<T>::SIZE == 2) {
    if (p.xs == 2) return launch_tiled_one<T, EPI, 2, false>(p, s);
  }
  return p.xs == 1 ? launch_tiled_one<T, EPI, 1, false>(p, s) : hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_tiled_t(int epi, const GemmParams &p, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: return launch_tiled_x<T, EPI_STORE>(p, s);
    case EPI_RESID: return launch_tiled_x<T, EPI_RESID>(p, s);
    case EPI_QKV: return launch_tiled_x<T, EPI_QKV>(p, s);
    case EPI_KVINJ: return launch_tiled_x<T, EPI_KVINJ>(p, s);
    case EPI_SWIGLU: return launch_tiled_x<T, EPI_SWIGLU>(p, s);
    case EPI_ARGMAX: return launch_tiled_x<T, EPI_ARGMAX>(p, s);
    case EPI_LOGITS: return launch_tiled_x<T, EPI_LOGITS>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_tiled(int dtype, int epi, const GemmParams &p, hipStream_t s) {
  return dtype == DFLASH_BF16 ? launch_tiled_t<bf16_t>(epi, p, s) : launch_tiled_t<float>(epi, p, s);
}

}  // namespace dflash
