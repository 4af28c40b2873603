// Y = X W^T on MFMA for launches with many rows (draft and verify GEMMs of
// more than 17 rows, injections of more than 32: the batched draft step and
// its heads, large injections).
//
// A workgroup owns a TM x TN tile of 16 x 16 output fragments (64 to 192
// tokens x 128 to 384 features, chosen per launch) and the whole K range or
// one of up to 8 parts of it; its 8 wavefronts form a 2 x 4 grid of
// sub-tiles, each accumulating (TM / 2) x (TN / 4) MFMA fragments.  Per 32-column k-tile the tile's activation fragments (TM row tiles, one
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

// Which tiled instantiations may split their k-tiles over workgroups: not the
// vocabulary-wide heads, and of the tiles with more than 8 fragments a
// wavefront only the plain stores (the others have no registers left for the
// exchange).  WM x WN: fragments a wavefront.
template <int EPI, int WM, int WN>
__host__ __device__ constexpr bool tl_can_split() {
  if (EPI == EPI_ARGMAX || EPI == EPI_LOGITS) return false;
  return WM * WN <= 8 || EPI == EPI_STORE || EPI == EPI_RESID;
}

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
  // Only these instantiations carry the split-K exchange (the launcher never
  // splits the others)
  constexpr bool SPLIT_CODE = tl_can_split<EPI, TM / WGM, TN / WGN>();
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
  constexpr bool ROPE = EPI == EPI_QKV || EPI == EPI_KVINJ;
  __shared__ double turns_s[ROPE ? MAX_ROPE_HALF : 1];
  __shared__ int ctx_s[ROPE ? MAX_SEQS : 1];
  __shared__ int cu_s[EPI == EPI_KVINJ ? MAX_SEQS + 1 : 1];
  __shared__ float rs_s[RS ? MAX_KEY_ROWS : 1];
  const bool rs_in_lds = RS && p.rs_direct && p.M <= MAX_KEY_ROWS;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int wm = wave / WGN, wn = wave % WGN;
  const int c = lane & 15, g = lane >> 4;
  const int K = p.k_tiles;
  // Work units: an item (feature block, token block) or, with ksplit > 1,
  // one of ksplit parts of its k-tile range.  XCD-aware order (the grid is a
  // multiple of 8): XCD x takes feature blocks x, x + 8, ...; its workgroups
  // walk those blocks' units with the part fastest, then the token block.
  // The vocabulary heads cap every workgroup at the grid's even share of
  // items: when the feature blocks do not split evenly over the XCDs, the few
  // items past the cap in the fuller XCDs go, in XCD order, to the workgroups
  // left below it (a weight block fetched once more, instead of a whole extra
  // round for one workgroup).  The other launches keep the plain dealing,
  // whose scalar registers they cannot spare.
  constexpr bool EVEN = EPI == EPI_ARGMAX || EPI == EPI_LOGITS;
  static_assert(!(EVEN && SPLIT_CODE), "the even dealing assumes unsplit items");
  const int xcd = int(blockIdx.x) % TL_XCDS, r = int(blockIdx.x) / TL_XCDS;
  const int per_xcd = int(gridDim.x) / TL_XCDS;
  const int ks = SPLIT_CODE ? p.ksplit : 1;
  const int per_nb = p.m_blocks * ks;
  auto units_in = [&](int x) { return (p.n_blocks - x + TL_XCDS - 1) / TL_XCDS * per_nb; };
  const int units_x = units_in(xcd);
  // unit index (item * ks + part) of XCD x's li-th unit
  auto unit_at = [&](int x, int li) { return (x + TL_XCDS * (li / per_nb)) * per_nb + li % per_nb; };
  int base = (units_x - r + per_xcd - 1) / per_xcd, my_items = base, spare_before = 0, cap = 0;
  if constexpr (EVEN) {
    cap = (p.n_blocks * per_nb + int(gridDim.x) - 1) / int(gridDim.x);
    const int q_x = units_x / per_xcd, rem_x = units_x % per_xcd;
    base = min(cap, q_x + (r < rem_x ? 1 : 0));
    // this workgroup's first slot among the grid's free slots (below the
    // cap), and the items past the cap over the grid
    spare_before = units_x < cap * per_xcd ? r * (cap - q_x) - min(r, rem_x) : 0;
    int over = 0;
    for (int x = 0; x < TL_XCDS; ++x) {
      const int u = units_in(x);
      over += max(0, u - cap * per_xcd);
      if (x < xcd) spare_before += max(0, cap * per_xcd - u);
    }
    my_items = base + min(cap - base, max(0, over - spare_before));
  }
  // unit index of this workgroup's i-th unit
  auto item_of = [&](int i) {
    if (!EVEN || i < base) return unit_at(xcd, r + i * per_xcd);
    int k = spare_before + (i - base);   // the k-th item past the cap
    int x = 0;
    for (; x < TL_XCDS - 1; ++x) {
      const int o = max(0, units_in(x) - cap * per_xcd);
      if (k < o) break;
      k -= o;
    }
    return unit_at(x, cap * per_xcd + k);
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

  // Epilogue.  A global load issued after a global store waits for that
  // store and for every stage load in flight before it (vector memory
  // counts retire in order), so each epilogue issues all of its global loads
  // (residual rows, norm gains, tree positions) in one batch before its
  // first store; the per-row scales, context lengths, segment bounds and
  // rotary frequencies come from LDS tables filled at kernel start.
  auto epilogue = [&](int item) {
    const int nblk = item / p.m_blocks, mblk = item % p.m_blocks;
    if constexpr (EPI == EPI_ARGMAX) {
      if (mblk != cur_mblk) {
        if (cur_mblk >= 0) flush_argmax(cur_mblk);
        cur_mblk = mblk;
      }
    }
    int m_a[TL_WM];
    bool mok_a[TL_WM];
    float rs_a[TL_WM];
#pragma unroll
    for (int a = 0; a < TL_WM; ++a) {
      m_a[a] = mblk * TL_MT * 16 + (wm * TL_WM + a) * 16 + c;
      mok_a[a] = m_a[a] < p.M;
      rs_a[a] = 1.f;
      if constexpr (RS) {
        if (p.rs_direct) rs_a[a] = !mok_a[a] ? 0.f : rs_in_lds ? rs_s[m_a[a]] : p.rs_direct[m_a[a]];
      }
    }
    if constexpr (EPI == EPI_ARGMAX) {
#pragma unroll
      for (int a = 0; a < TL_WM; ++a) {
        const int ml = (wm * TL_WM + a) * 16 + c;
        unsigned long long k = 0;
#pragma unroll
        for (int b = 0; b < TL_WN; ++b) {
          const int n0 = (nblk * TL_NT + wn * TL_WN + b) * 16 + 4 * g;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (n0 + i < p.vocab) {
              const unsigned long long kk = argmax_key(acc[a][b][i] * rs_a[a], n0 + i);
              k = kk > k ? kk : k;
            }
          }
        }
        unsigned long long o = __shfl_xor(k, 16, 64);
        k = o > k ? o : k;
        o = __shfl_xor(k, 32, 64);
        k = o > k ? o : k;
        if (g == 0 && mok_a[a]) __hip_atomic_fetch_max(best_row + ml, k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    } else if constexpr (EPI == EPI_LOGITS) {
#pragma unroll
      for (int a = 0; a < TL_WM; ++a)
#pragma unroll
        for (int b = 0; b < TL_WN; ++b) {
          const int n0 = (nblk * TL_NT + wn * TL_WN + b) * 16 + 4 * g;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (mok_a[a] && n0 + i < p.vocab) p.out_f32[size_t(m_a[a]) * p.ld_out + n0 + i] = acc[a][b][i] * rs_a[a];
        }
    } else if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int a = 0; a < TL_WM; ++a)
#pragma unroll
        for (int b = 0; b < TL_WN; b += 2) {
          const int pair = (nblk * TL_NT + wn * TL_WN + b) >> 1;
          f32x4 out = f32x4{0.f, 0.f, 0.f, 0.f};
          if (mok_a[a]) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float gt = acc[a][b][i] * rs_a[a], up = acc[a][b + 1][i] * rs_a[a];
              out[i] = gt / (1.0f + __expf(-gt)) * up;
            }
          }
          if (m_a[a] < p.x_mtiles * 16 && pair < p.n_tiles / 2)  // padded rows get zeros
            store_split4<T>(p.out_packed + packed_offset<T>(m_a[a], pair * 16 + 4 * g, p.out_kt), p.out_plane,
                            p.out_planes, out);
        }
    } else if constexpr (EPI == EPI_STORE || EPI == EPI_RESID) {
      // Rows A0 .. A0 + NA - 1 of the wavefront's fragments: loads first
      // (residual fragments, the next norm's gains), then the values (zero
      // outside the output), their stores and the tile sums.  Small tiles
      // take every row in one pass; large ones (no registers for all the
      // residual fragments at once) one row of fragments at a time.
      constexpr int NA = TL_WM * TL_WN <= 8 ? TL_WM : 1;
      f32x4 gain[TL_WN];
#pragma unroll
      for (int b = 0; b < TL_WN; ++b) {
        const int ntg = nblk * TL_NT + wn * TL_WN + b;
        const int n0 = ntg * 16 + 4 * g;
        gain[b] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (p.nx_packed && ntg < p.n_tiles) {
          if constexpr (ES == 2) {
            const uint2 w = *reinterpret_cast<const uint2 *>(p.nx_gain + size_t(n0) * 2);
            gain[b] = f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
                            __uint_as_float(w.y & 0xffff0000u)};
          } else {
            gain[b] = *reinterpret_cast<const f32x4 *>(p.nx_gain + size_t(n0) * 4);
          }
        }
      }
#pragma unroll
      for (int A0 = 0; A0 < TL_WM; A0 += NA) {
        f32x4 val[NA][TL_WN];
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
          for (int b = 0; b < TL_WN; ++b) {
            const int ntg = nblk * TL_NT + wn * TL_WN + b;
            val[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
            if constexpr (EPI == EPI_RESID) {
              if (mok_a[A0 + a] && ntg < p.n_tiles)
                val[a][b] = *reinterpret_cast<const f32x4 *>(p.resid + size_t(m_a[A0 + a]) * p.ld_out + ntg * 16 + 4 * g);
            }
          }
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
          for (int b = 0; b < TL_WN; ++b) {
            const bool ok = mok_a[A0 + a] && nblk * TL_NT + wn * TL_WN + b < p.n_tiles;
            f32x4 v = acc[A0 + a][b] * rs_a[A0 + a];
            if constexpr (EPI == EPI_RESID) v += val[a][b];
            val[a][b] = ok ? v : f32x4{0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
        for (int a = 0; a < NA; ++a)
#pragma unroll
          for (int b = 0; b < TL_WN; ++b) {
            const int ntg = nblk * TL_NT + wn * TL_WN + b;
            const int n0 = ntg * 16 + 4 * g;
            const int m = m_a[A0 + a];
            if (mok_a[A0 + a] && ntg < p.n_tiles) {
              *reinterpret_cast<f32x4 *>(p.out_f32 + size_t(m) * p.ld_out + n0) = val[a][b];
              if (p.aux_out) {
#pragma unroll
                for (int i = 0; i < 4; ++i) store_elem<T>(p.aux_out + (size_t(m) * p.aux_ld + n0 + i) * ES, val[a][b][i]);
              }
            }
            if (p.nx_packed && ntg < p.n_tiles && m < p.nx_rows)
              store_split4<T>(p.nx_packed + packed_offset<T>(m, n0, p.nx_kt), p.nx_plane, p.nx_planes, val[a][b] * gain[b]);
          }
        if (p.ssq_out) {
          // the balanced tree of tile_ssq16: in-lane pairs, then g ^ 1, g ^ 2
#pragma unroll
          for (int a = 0; a < NA; ++a)
#pragma unroll
            for (int b = 0; b < TL_WN; ++b) {
              const f32x4 v = val[a][b];
              float q = (__fmul_rn(v[0], v[0]) + __fmul_rn(v[1], v[1])) + (__fmul_rn(v[2], v[2]) + __fmul_rn(v[3], v[3]));
              q += __shfl_xor(q, 16, 64);
              q += __shfl_xor(q, 32, 64);
              const int ntg = nblk * TL_NT + wn * TL_WN + b;
              if (g == 0 && mok_a[A0 + a] && ntg < p.n_tiles) p.ssq_out[size_t(m_a[A0 + a]) * p.ssq_ld + ntg] = q;
            }
        }
      }
    } else if constexpr (EPI == EPI_QKV) {
      // A lane's four features n0 .. n0 + 3 of a fragment are four
      // consecutive channels of one head in the packed rotary order, so the
      // q and k rows take one store per lane chunk; v (position-interleaved
      // layout) takes one per element.
      const int d = p.head_dim, nqd = p.n_q * d, nkd = p.n_kv * d;
      const int dt_count = d / KT;
      int rp[TL_WM];   // rotary position offset of each row: its tree depth, else its block slot
#pragma unroll
      for (int a = 0; a < TL_WM; ++a) rp[a] = p.row_pos && mok_a[a] ? p.row_pos[m_a[a]] : m_a[a] % p.block;
#pragma unroll
      for (int a = 0; a < TL_WM; ++a) {
        const int m = m_a[a];
        const int sq = m / p.block, j = m % p.block;
        const int ctx = mok_a[a] ? ctx_s[min(sq, MAX_SEQS - 1)] : 0;
#pragma unroll
        for (int b = 0; b < TL_WN; ++b) {
          const int ntg = nblk * TL_NT + wn * TL_WN + b;
          const int n0 = ntg * 16 + 4 * g;
          const f32x4 v = acc[a][b] * rs_a[a];
          f32x4 partner;   // features n ^ 8: lane g ^ 2
#pragma unroll
          for (int i = 0; i < 4; ++i) partner[i] = __shfl_xor(v[i], 32, 64);
          if (!(mok_a[a] && ntg < p.n_tiles)) continue;
          if (n0 < nqd + nkd) {
            const int dd0 = rot_channel(n0 % d, d);
            f32x4 x = v;
            if (p.rope_on) {
#pragma unroll
              for (int i = 0; i < 4; ++i)
                x[i] = rope_rotate(v[i], partner[i], dd0 + i, d, ctx + rp[a], turns_s[(dd0 + i) % (d >> 1)]);
            }
            if (n0 < nqd) {
              char *base = p.qbuf + (size_t(sq) * p.n_q + n0 / d) * p.q_tiles * dt_count * 1024;
              store_split4<T>(base + packed_offset<T>(j, dd0, dt_count), p.q_plane, p.q_planes, x);
            } else {
              char *base = p.kblk + (size_t(sq) * p.n_kv + (n0 - nqd) / d) * size_t(KT) * d * ES;
              store_elem4<T>(base + kcache_offset<T>(j, dd0, d), x);
              if (p.qkv_to_cache) qkv_cache_store_k4<T>(p, sq, (n0 - nqd) / d, ctx + j, dd0, x);
            }
          } else {
            const int cc0 = n0 - nqd - nkd;
            char *base = p.vblk + (size_t(sq) * p.n_kv + cc0 / d) * size_t(KT) * d * ES;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              store_elem<T>(base + vcache_offset<T>(j, cc0 % d + i, d), v[i]);
              if (p.qkv_to_cache) qkv_cache_store<T>(p, false, sq, cc0 / d, ctx + j, cc0 % d + i, v[i]);
            }
          }
        }
      }
    } else if constexpr (EPI == EPI_KVINJ) {
      const int d = p.head_dim, nkd = p.n_kv * d, segn = 2 * nkd;
      const size_t region = size_t(p.capacity) * d * ES;
#pragma unroll
      for (int a = 0; a < TL_WM; ++a) {
        const int m = m_a[a];
        const bool mok = mok_a[a];
        int sq = 0, start = 0, ns = 0, C = 0;
        if (mok) {
          int lo = 0, hi = p.batch;  // cu_new[lo] <= m < cu_new[lo + 1]
          while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (cu_s[mid] <= m) lo = mid; else hi = mid;
          }
          sq = lo;
          start = cu_s[sq];
          ns = cu_s[sq + 1] - start;
          C = ctx_s[sq];
        }
        const bool fits = C + ns <= p.capacity;
#pragma unroll
        for (int b = 0; b < TL_WN; ++b) {
          const int ntg = nblk * TL_NT + wn * TL_WN + b;
          const int n0 = ntg * 16 + 4 * g;
          const bool nok = ntg < p.n_tiles;
          const f32x4 v = acc[a][b] * rs_a[a];
          f32x4 partner;
#pragma unroll
          for (int i = 0; i < 4; ++i) partner[i] = __shfl_xor(v[i], 32, 64);
          if (!(mok && nok)) continue;
          if (!fits) {
            if (m == start && n0 == 0) atomicOr(p.status, DFLASH_STATUS_CAPACITY);
            continue;
          }
          const int pos = C + (m - start);
          const int layer = p.layer0 + n0 / segn, cc0 = n0 % segn;
          if (cc0 < nkd) {
            const int dd0 = rot_channel(cc0 % d, d);
            f32x4 r = v;
            if (p.rope_on) {
#pragma unroll
              for (int i = 0; i < 4; ++i)
                r[i] = rope_rotate(v[i], partner[i], dd0 + i, d, pos, turns_s[(dd0 + i) % (d >> 1)]);
            }
            char *base = p.kcache + ((size_t(layer) * p.max_batch + sq) * p.n_kv + cc0 / d) * region;
            store_elem4<T>(base + kcache_offset<T>(pos, dd0, d), r);
          } else {
            const int c2 = cc0 - nkd;
            char *base = p.vcache + ((size_t(layer) * p.max_batch + sq) * p.n_kv + c2 / d) * region;
#pragma unroll
            for (int i = 0; i < 4; ++i) store_elem<T>(base + vcache_offset<T>(pos, c2 % d + i, d), v[i]);
          }
        }
      }
    }
    zero();
  };

  if constexpr (EPI == EPI_ARGMAX) {
    if (int(threadIdx.x) < TL_MT * 16) best_row[threadIdx.x] = 0;
  }
  // The epilogue's small tables, read before any stage is issued (so the
  // wait for them is one round trip, not a drain of the ring).
  if constexpr (ROPE) {
    if (wave == 0) {
      double v = 0.0;
#pragma unroll
      for (int i = 0; i < MAX_ROPE_HALF; ++i) v = lane == i ? p.rope_turns[i] : v;   // kernel-argument reads
      turns_s[lane] = v;
    }
    const int nseq = EPI == EPI_KVINJ ? p.batch : min((p.M + p.block - 1) / p.block, MAX_SEQS);
    for (int i = threadIdx.x; i < nseq; i += blockDim.x) ctx_s[i] = p.ctx_len[i];
    if constexpr (EPI == EPI_KVINJ) {
      for (int i = threadIdx.x; i <= p.batch; i += blockDim.x) cu_s[i] = p.cu_new[i];
    }
  }
  if constexpr (RS) {
    if (rs_in_lds) {
      for (int i = threadIdx.x; i < p.M; i += blockDim.x) rs_s[i] = p.rs_direct[i];
    }
  }
  __syncthreads();
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
  // tile (16-byte agent-coherent stores, one f32x4 per lane and fragment),
  // waits for them and counts itself in; the last to arrive sums the parts
  // in part order from the workspace, so the result does not depend on
  // which part finished last, resets the count and runs the epilogue.
  auto split_last = [&](int unit) -> bool {
    const int item = unit / ks;
    // A unit's partial tile: per wavefront its TL_WM x TL_WN fragments, 1 KiB
    // each, one 16-byte run per lane; the unit and wavefront part of the
    // offset is uniform.
    constexpr int FR = TL_WM * TL_WN;
    const auto prs = __builtin_amdgcn_make_buffer_rsrc(p.part_ws, (short)0, int(SPLIT_PART_BYTES), BUF_DWORD3);
    auto base_of = [&](int u) { return __builtin_amdgcn_readfirstlane((u * TL_WAVES + wave) * FR * 1024); };
    const int lane_off = lane * 16;
    {
      const int sb = base_of(unit);
#pragma unroll
      for (int a = 0; a < TL_WM; ++a)
#pragma unroll
        for (int b = 0; b < TL_WN; ++b) st16_agent(prs, lane_off + (a * TL_WN + b) * 1024, sb, acc[a][b]);
    }
    if (!last_arriver_of(p.part_cnt + item, unsigned(ks), &flag)) {
      zero();
      return false;
    }
    if (threadIdx.x == 0) __hip_atomic_store(p.part_cnt + item, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // Small tiles: GP parts' loads in flight together (16 fragments a
    // wavefront), summed in part order; a group past the last part reloads
    // the last part and drops it.  Large tiles: one part at a time, a row of
    // fragments per load group.
    if constexpr (FR <= 8) {
      constexpr int GP = 16 / FR;
      for (int j0 = 0; j0 < ks; j0 += GP) {
        f32x4 v[GP][TL_WM][TL_WN];
#pragma unroll
        for (int q = 0; q < GP; ++q) {
          const int sb = base_of(item * ks + min(j0 + q, ks - 1));
#pragma unroll
          for (int a = 0; a < TL_WM; ++a)
#pragma unroll
            for (int b = 0; b < TL_WN; ++b) v[q][a][b] = ld16_agent(prs, lane_off + (a * TL_WN + b) * 1024, sb);
        }
#pragma unroll
        for (int q = 0; q < GP; ++q) {
          if (j0 + q < ks) {
#pragma unroll
            for (int a = 0; a < TL_WM; ++a)
#pragma unroll
              for (int b = 0; b < TL_WN; ++b) acc[a][b] = j0 + q == 0 ? v[q][a][b] : acc[a][b] + v[q][a][b];
          }
        }
      }
    } else {
      for (int j = 0; j < ks; ++j) {
        const int sb = base_of(item * ks + j);
#pragma unroll
        for (int a = 0; a < TL_WM; ++a) {
          f32x4 v[TL_WN];
#pragma unroll
          for (int b = 0; b < TL_WN; ++b) v[b] = ld16_agent(prs, lane_off + (a * TL_WN + b) * 1024, sb);
#pragma unroll
          for (int b = 0; b < TL_WN; ++b) acc[a][b] = j == 0 ? v[b] : acc[a][b] + v[b];
        }
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
    bool run_epi = true;
    if constexpr (SPLIT_CODE) run_epi = ks == 1 || split_last(unit);
    if (run_epi) epilogue(unit / ks);
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

// Tile and split choice of the non-head launches.  The kernel is bound by
// staging fragments through LDS, so a choice costs its busiest workgroup's
// 1 KiB fragment loads (per k-tile: the tile's activation fragments, one or
// two planes, and its weight fragments), weighted by how few ring stages the
// tile leaves in flight (measured per fragment: 9 stages 1.0, 6 about 1.1,
// 4 about 1.15, 3 about 1.25), plus about 100 fragments' time per unit for
// its epilogue and, for split items, about 120 more per unit for storing its
// partial tile and counting in and about 50 per round trip of the last
// part's gather.  Tiles: 64 x 128 for every epilogue; 64 x 192 for
// QKV (its rotary partner exchange does not fit a 128-row tile); 64 x 256
// and 128 x 256 for the others; 128 x 384 for gate/up.  k-tiles split into
// at most 8 parts of at least 8 when the workspace holds the partial tiles;
// a split must beat the unsplit choices by 10%, about the model's error
// against the kernel times it was fitted to.
struct TileChoice {
  int tm, tn, ks;
};
template <int EPI, int XS>
static TileChoice choose_tile(int M, int n_tiles, int k_tiles, int cu, bool split_ws) {
  auto blocks = [](long n, long b) { return (n + b - 1) / b; };
  TileChoice best{4, 8, 1};
  long best_cost = -1;
  auto consider = [&](int tm, int tn, bool splittable) {
    const long mb = blocks(M, 16 * tm), nb = blocks(n_tiles, tn);
    const int fr = (tm / 2) * (tn / 4);   // fragments a wavefront
    for (int ks = 1; ks <= 8; ++ks) {
      if (ks > 1 && !(splittable && split_ws && k_tiles / ks >= 8)) break;
      const long units = mb * nb * ks;
      if (ks > 1 && (units * tm * tn * 1024 > long(SPLIT_PART_BYTES) || mb * nb > MAX_SPLIT_ITEMS)) break;
      long grid = units < cu ? units : cu;
      grid = grid < TL_XCDS ? TL_XCDS : grid - grid % TL_XCDS;
      const long per_wg = blocks(blocks(nb, TL_XCDS) * mb * ks, grid / TL_XCDS);   // the busiest XCD's share
      const long rounds = ks == 1 ? 0 : fr <= 8 ? blocks(ks, 16 / fr) + 2 : long(ks) * (tm / 2) + 2;
      const long stages = 144 / (blocks(XS * tm + tn, 8) * 8);
      const long weight = stages >= 8 ? 100 : stages >= 6 ? 110 : stages >= 4 ? 115 : 125;   // percent
      long cost = per_wg * (blocks(k_tiles, ks) * (XS * tm + tn) * weight / 100 + 100 + (ks > 1 ? 120 : 0)) +
                  50 * rounds;
      if (ks > 1) cost += cost / 10;   // a split must win by a margin the model can resolve
      if (best_cost < 0 || cost < best_cost) {
        best_cost = cost;
        best = TileChoice{tm, tn, ks};
      }
    }
  };
  consider(4, 8, tl_can_split<EPI, 2, 2>());
  if constexpr (EPI == EPI_QKV) {
    consider(4, 12, tl_can_split<EPI, 2, 3>());
  } else {
    consider(4, 16, tl_can_split<EPI, 2, 4>());
    consider(8, 16, tl_can_split<EPI, 4, 4>());
    if constexpr (EPI == EPI_SWIGLU) consider(8, 24, tl_can_split<EPI, 4, 6>());
  }
  return best;
}

// Tile choice, 8 wavefronts in a 2 x 4 grid:
//   heads (argmax): TM x 16 fragments with TM even, at most 12: one token
//     block covering every row when it fits (each weight byte read once),
//     else 8 or 12, whichever pads the rows less; the TM = 8 head with one
//     activation plane is 24 fragments wide, and so are the TM = 4 and 6
//     heads when that takes fewer rounds of items on the compute units (a
//     full round streams at the chip's HBM rate whatever the width, a short
//     last round is bound by the k-step chain, so a round saved is worth it);
//   others: by choose_tile.
template <typename T, int EPI, int XS, bool XROW>
static hipError_t launch_tiled_one(const GemmParams &p0, hipStream_t s) {
  GemmParams p = p0;
  const int cu = p.grid_cap;
  auto blocks = [](int n, int b) { return (n + b - 1) / b; };
  const int mt = blocks(p.M, 16);
  constexpr bool HEAD = EPI == EPI_ARGMAX || EPI == EPI_LOGITS;   // vocabulary-wide heads
  int tn = 16;
  p.ksplit = 1;
  if (HEAD) {
    // at least 4 fragments: 2 (17-32 rows) would leave half the wave grid
    // without a row tile
    if (mt <= 12) p.tile_m = mt <= 4 ? 4 : (mt + 1) & ~1;
    else p.tile_m = blocks(mt, 12) * 12 < blocks(mt, 8) * 8 ? 12 : 8;
    // the 128-row head tile is 384 features wide (one plane of activations
    // leaves the registers for it; at 10 and 12 fragments that width spills):
    // each staged weight fragment feeds more MFMAs
    bool wide = XS == 1 && p.tile_m == 8;
    if (XS == 1 && (p.tile_m == 4 || p.tile_m == 6)) {
      // items of the busiest workgroup at width tn (heads deal their items
      // evenly over the grid)
      auto rounds = [&](int tn_) {
        const int items_ = blocks(p.M, 16 * p.tile_m) * blocks(p.n_tiles, tn_);
        int g = items_ < cu ? items_ : cu;
        g = g < TL_XCDS ? TL_XCDS : g - g % TL_XCDS;
        return blocks(items_, g);
      };
      wide = rounds(24) < rounds(16);
    }
    p.n_blocks = blocks(p.n_tiles, wide ? 24 : 16);
    tn = wide ? 24 : 16;
  } else {
    const TileChoice tc = choose_tile<EPI, XS>(p.M, p.n_tiles, p.k_tiles, cu, p.part_ws && p.part_cnt);
    p.tile_m = tc.tm;
    p.n_blocks = blocks(p.n_tiles, tc.tn);
    p.ksplit = tc.ks;
    tn = tc.tn;
  }
  p.m_blocks = blocks(p.M, 16 * p.tile_m);
  const int items = p.m_blocks * p.n_blocks;
  // grid: a multiple of the 8 XCDs, at most one workgroup per compute unit
  const int units = items * p.ksplit;
  int grid = units < cu ? units : cu;
  grid = grid < TL_XCDS ? TL_XCDS : grid - grid % TL_XCDS;
  if constexpr (HEAD && XS == 1) {
    switch (p.tile_m) {
      case 4:
        if (tn == 24) launch_tiled_shape<T, EPI, XS, XROW, 4, 24, 2, 4>(p, grid, s);
        else launch_tiled_shape<T, EPI, XS, XROW, 4, 16, 2, 4>(p, grid, s);
        break;
      case 6:
        if (tn == 24) launch_tiled_shape<T, EPI, XS, XROW, 6, 24, 2, 4>(p, grid, s);
        else launch_tiled_shape<T, EPI, XS, XROW, 6, 16, 2, 4>(p, grid, s);
        break;
      case 8: launch_tiled_shape<T, EPI, XS, XROW, 8, 24, 2, 4>(p, grid, s); break;
      case 10: launch_tiled_shape<T, EPI, XS, XROW, 10, 16, 2, 4>(p, grid, s); break;
      case 12: launch_tiled_shape<T, EPI, XS, XROW, 12, 16, 2, 4>(p, grid, s); break;
      default: return hipErrorInvalidValue;
    }
  } else if constexpr (HEAD) {
    if (p.tile_m != 8) return hipErrorInvalidValue;
    launch_tiled_shape<T, EPI, XS, XROW, 8, 16, 2, 4>(p, grid, s);
  } else {
    const int shape = p.tile_m * 100 + tn;
    if (shape == 408) {
      launch_tiled_shape<T, EPI, XS, XROW, 4, 8, 2, 4>(p, grid, s);
      return hipGetLastError();
    }
    if constexpr (EPI == EPI_QKV) {
      if (shape == 412) {
        launch_tiled_shape<T, EPI, XS, XROW, 4, 12, 2, 4>(p, grid, s);
        return hipGetLastError();
      }
    } else {
      if (shape == 416) {
        launch_tiled_shape<T, EPI, XS, XROW, 4, 16, 2, 4>(p, grid, s);
        return hipGetLastError();
      }
      if (shape == 816) {
        launch_tiled_shape<T, EPI, XS, XROW, 8, 16, 2, 4>(p, grid, s);
        return hipGetLastError();
      }
      if constexpr (EPI == EPI_SWIGLU) {
        if (shape == 824) {
          launch_tiled_shape<T, EPI, XS, XROW, 8, 24, 2, 4>(p, grid, s);
          return hipGetLastError();
        }
      }
    }
    return hipErrorInvalidValue;
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
