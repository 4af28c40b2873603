// Y = X W^T on MFMA for the skinny shapes of a draft step (M = 16 rows per
// sequence), with split-K and fused epilogues.
//
// Operands are packed fragment tiles (1 KiB = one 64-lane MFMA operand), so
// every wavefront load is a single coalesced 1 KiB read.  The weight tile is
// the A operand (rows = output features) and the activation tile the B
// operand (rows = tokens); lane (c, g) of an accumulator then holds token c
// and output features 4g..4g+3.  A workgroup owns NB 16-column weight tiles
// and MT 16-row token tiles; its four wavefronts split the workgroup's K
// range and add their partial sums in LDS in a fixed order.  When K is split
// over workgroups, partial tiles go to the workspace and the last-arriving
// workgroup of a tile adds them in split order and runs the epilogue, so the
// result does not depend on scheduling.
#include "common.hpp"
#include "kernels.hpp"

namespace dflash {

__device__ inline float tile_at(const f32x4 *t, int NB, int ml, int nl) {
  const int f = (ml >> 4) * NB + (nl >> 4);
  const int ln = (ml & 15) + 16 * ((nl & 15) >> 2);
  return t[f * 64 + ln][nl & 3];
}

// cos and sin of pos * theta^(-2i/d), evaluated in fp64 and rounded once.
__device__ inline void rope_cs(int pos, int i, int d, float theta, float *c, float *s) {
  const double inv = pow(double(theta), -2.0 * double(i) / double(d));
  const double a = double(pos) * inv;
  double sd, cd;
  sincos(a, &sd, &cd);
  *c = float(cd);
  *s = float(sd);
}

__device__ inline float rope_apply(float v, float partner, int dd, int d, int pos, float theta) {
  if (theta == 0.f) return v;
  const int half = d >> 1;
  float c, s;
  rope_cs(pos, dd % half, d, theta, &c, &s);
  return dd < half ? v * c - partner * s : v * c + partner * s;
}

template <typename T> __device__ inline void store_elem(char *p, float v);
template <> __device__ inline void store_elem<float>(char *p, float v) { *reinterpret_cast<float *>(p) = v; }
template <> __device__ inline void store_elem<bf16_t>(char *p, float v) {
  *reinterpret_cast<uint16_t *>(p) = f32_to_bf16(v);
}

// Orderable 64-bit key: larger value first, then lower index.
__device__ inline unsigned long long argmax_key(float v, int n) {
  if (v == 0.0f) v = 0.0f;  // -0 and +0 compare equal
  unsigned u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<unsigned long long>(u) << 32) | static_cast<unsigned>(~static_cast<unsigned>(n));
}

__device__ inline int key_index(unsigned long long k) {
  return static_cast<int>(~static_cast<unsigned>(k & 0xffffffffull));
}

template <typename T, int MT, int NB, int EPI, int XS>
__global__ __launch_bounds__(256) void gemm_kernel(const GemmParams p) {
  constexpr int E = Ty<T>::E, KT = Ty<T>::KT, ES = Ty<T>::SIZE;
  constexpr int U = (MT * XS) >= 4 ? 2 : 4;
  constexpr int NF = MT * NB;
  constexpr int R = MT * 16, CN = NB * 16;
  __shared__ f32x4 red[4 * NF * 64];
  __shared__ int s_flag;

  const int total = p.m_blocks * p.n_blocks * p.splits;
  const int bid = xcd_remap(blockIdx.x, total);
  const int split = bid % p.splits;
  const int t2 = bid / p.splits;
  const int nblk = t2 % p.n_blocks;
  const int mblk = t2 / p.n_blocks;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;

  const int nt0 = nblk * NB;
  const int seg = nt0 / p.seg_ntiles;
  const char *wbase = p.w_seg[seg] + size_t(nt0 - seg * p.seg_ntiles) * p.k_tiles * 1024 + lane * 16;
  const size_t wstride = size_t(p.k_tiles) * 1024;

  const int kb = split * p.kt_per_split;
  const int ke = min(kb + p.kt_per_split, p.k_tiles);
  const int per = (ke - kb + 3) >> 2;
  const int k0 = kb + wave * per;
  const int k1 = min(k0 + per, ke);
  const int mt0 = mblk * MT;

  // B-operand chunk of token tile mt at column tile kt, activation plane xp
  // (zero past the rows).
  auto load_x = [&](int mt, int kt, int xp) -> uint4 {
    const int mtg = mt0 + mt;
    if (p.x_ld == 0) {
      if (mtg >= p.m_tiles) return make_uint4(0, 0, 0, 0);
      return ld16(p.x + xp * p.x_plane + (size_t(mtg) * p.k_tiles + kt) * 1024 + lane * 16);
    }
    const int row = mtg * 16 + (lane & 15);
    if (row >= p.M) return make_uint4(0, 0, 0, 0);
    const int col = kt * KT + (lane >> 4) * E;
    return ld16(p.x + (size_t(row) * p.x_ld + col) * ES);
  };

  f32x4 acc[MT][NB];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mt][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  int kt = k0;
  for (; kt + U <= k1; kt += U) {
    uint4 wf[U][NB], xf[U][MT][XS];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) wf[u][nb] = ld16_stream(wbase + nb * wstride + size_t(kt + u) * 1024);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int xp = 0; xp < XS; ++xp) xf[u][mt][xp] = load_x(mt, kt + u, xp);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int xp = 0; xp < XS; ++xp) acc[mt][nb] = mma<T>(acc[mt][nb], wf[u][nb], xf[u][mt][xp]);
  }
  for (; kt < k1; ++kt) {
    uint4 wf[NB], xf[MT][XS];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) wf[nb] = ld16_stream(wbase + nb * wstride + size_t(kt) * 1024);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int xp = 0; xp < XS; ++xp) xf[mt][xp] = load_x(mt, kt, xp);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int xp = 0; xp < XS; ++xp) acc[mt][nb] = mma<T>(acc[mt][nb], wf[nb], xf[mt][xp]);
  }

  // Sum the four wavefronts' partial tiles in a fixed order.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) red[(wave * NF + mt * NB + nb) * 64 + lane] = acc[mt][nb];
  __syncthreads();
  for (int e = threadIdx.x; e < NF * 64; e += 256) {
    f32x4 s = red[e];
    s += red[NF * 64 + e];
    s += red[2 * NF * 64 + e];
    s += red[3 * NF * 64 + e];
    red[e] = s;
  }

  if (p.splits > 1) {
    const int tile_id = mblk * p.n_blocks + nblk;
    f32x4 *part = reinterpret_cast<f32x4 *>(p.partial) + size_t(tile_id) * p.splits * NF * 64;
    for (int e = threadIdx.x; e < NF * 64; e += 256) part[size_t(split) * NF * 64 + e] = red[e];
    if (!arrive_last(p.counters + CNT_TILE + tile_id, p.splits, &s_flag)) return;
    for (int e = threadIdx.x; e < NF * 64; e += 256) {
      f32x4 s = part[e];
      for (int z = 1; z < p.splits; ++z) s += part[size_t(z) * NF * 64 + e];
      red[e] = s;
    }
  }
  __syncthreads();

  // ---------------------------------------------------------------- epilogues
  if constexpr (EPI == EPI_STORE || EPI == EPI_RESID) {
    for (int e = threadIdx.x; e < R * CN; e += 256) {
      const int ml = e / CN, nl = e % CN;
      const int m = mblk * R + ml, n = nblk * CN + nl;
      if (m >= p.M || n >= p.N) continue;
      float v = tile_at(red, NB, ml, nl);
      const size_t o = size_t(m) * p.ld_out + n;
      if constexpr (EPI == EPI_RESID) v += p.resid[o];
      p.out_f32[o] = v;
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    constexpr int HALF = NB / 2;
    for (int e = threadIdx.x; e < R * HALF * 16; e += 256) {
      const int ml = e / (HALF * 16), q = e % (HALF * 16);
      const int pr = q >> 4, c = q & 15;
      const int m = mblk * R + ml;
      if (m >= p.m_tiles * 16) continue;
      const int col = (nblk * HALF + pr) * 16 + c;
      float out = 0.f;
      if (m < p.M) {
        const float gt = tile_at(red, NB, ml, 2 * pr * 16 + c);
        const float up = tile_at(red, NB, ml, (2 * pr + 1) * 16 + c);
        out = gt / (1.0f + __expf(-gt)) * up;
      }
      store_split<T>(p.out_packed + packed_offset<T>(m, col, p.out_kt), p.out_plane, p.out_planes, out);
    }
  } else if constexpr (EPI == EPI_QKV) {
    const int d = p.head_dim, nqd = p.n_q * d, nkd = p.n_kv * d;
    const int dt_count = d / KT;
    for (int e = threadIdx.x; e < R * CN; e += 256) {
      const int ml = e / CN, nl = e % CN;
      const int m = mblk * R + ml, n = nblk * CN + nl;
      if (m >= p.M) continue;
      const int s = m / p.block, j = m % p.block;
      float v = tile_at(red, NB, ml, nl);
      if (n < nqd + nkd) {
        const int dd = rot_channel(n % d, d);
        const int pos = p.ctx_len[s] + j;
        v = rope_apply(v, tile_at(red, NB, ml, nl ^ 8), dd, d, pos, p.rope_theta);
        if (n < nqd) {
          const int h = n / d;
          char *base = p.qbuf + (size_t(s) * p.n_q + h) * dt_count * 1024;
          store_split<T>(base + packed_offset<T>(j, dd, dt_count), p.q_plane, p.xs, v);
        } else {
          const int g = (n - nqd) / d;
          char *base = p.kblk + (size_t(s) * p.n_kv + g) * size_t(KT) * d * ES;
          store_elem<T>(base + kcache_offset<T>(j, dd, d), v);
        }
      } else {
        const int c = n - nqd - nkd;
        const int g = c / d, dd = c % d;
        char *base = p.vblk + (size_t(s) * p.n_kv + g) * size_t(KT) * d * ES;
        store_elem<T>(base + vcache_offset<T>(j, dd, d), v);
      }
    }
  } else if constexpr (EPI == EPI_KVINJ) {
    const int d = p.head_dim, nkd = p.n_kv * d, segn = 2 * nkd;
    const size_t region = size_t(p.capacity) * d * ES;
    int *ctx_len = const_cast<int *>(p.ctx_len);
    for (int e = threadIdx.x; e < R * CN; e += 256) {
      const int ml = e / CN, nl = e % CN;
      const int m = mblk * R + ml, n = nblk * CN + nl;
      if (m >= p.M) continue;
      int lo = 0, hi = p.batch;  // find s with cu_new[s] <= m < cu_new[s+1]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.cu_new[mid] <= m) lo = mid; else hi = mid;
      }
      const int s = lo, start = p.cu_new[s], ns = p.cu_new[s + 1] - start;
      const int C = ctx_len[s];
      if (C + ns > p.capacity) {
        if (m == start && n == 0) atomicOr(p.status, DFLASH_STATUS_CAPACITY);
        continue;
      }
      const int pos = C + (m - start);
      const int layer = p.layer0 + n / segn, c = n % segn;
      const float v = tile_at(red, NB, ml, nl);
      if (c < nkd) {
        const int g = c / d, dd = rot_channel(c % d, d);
        const float r = rope_apply(v, tile_at(red, NB, ml, nl ^ 8), dd, d, pos, p.rope_theta);
        char *base = p.kcache + ((size_t(layer) * p.max_batch + s) * p.n_kv + g) * region;
        store_elem<T>(base + kcache_offset<T>(pos, dd, d), r);
      } else {
        const int c2 = c - nkd, g = c2 / d, dd = c2 % d;
        char *base = p.vcache + ((size_t(layer) * p.max_batch + s) * p.n_kv + g) * region;
        store_elem<T>(base + vcache_offset<T>(pos, dd, d), v);
      }
    }
    if (arrive_last(p.counters + CNT_FINAL, p.m_blocks * p.n_blocks, &s_flag)) {
      for (int s = threadIdx.x; s < p.batch; s += 256) {
        const int ns = p.cu_new[s + 1] - p.cu_new[s];
        if (ctx_len[s] + ns <= p.capacity) ctx_len[s] += ns;
      }
    }
  } else if constexpr (EPI == EPI_ARGMAX) {
    if (threadIdx.x < R) {
      const int ml = threadIdx.x;
      unsigned long long best = 0;
      for (int nl = 0; nl < CN; ++nl) {
        const int n = nblk * CN + nl;
        if (n < p.vocab) {
          const unsigned long long k = argmax_key(tile_at(red, NB, ml, nl), n);
          best = k > best ? k : best;
        }
      }
      p.lvl1[(size_t(mblk) * p.n_blocks + nblk) * R + ml] = best;
    }
    const int grp = nblk / ARGMAX_GROUP;
    const int gsz = min(ARGMAX_GROUP, p.n_blocks - grp * ARGMAX_GROUP);
    if (!arrive_last(p.counters + CNT_GROUP + mblk * p.n_groups + grp, gsz, &s_flag)) return;
    if (threadIdx.x < R) {
      const int ml = threadIdx.x;
      unsigned long long best = 0;
      for (int i = 0; i < gsz; ++i) {
        const unsigned long long k = p.lvl1[(size_t(mblk) * p.n_blocks + grp * ARGMAX_GROUP + i) * R + ml];
        best = k > best ? k : best;
      }
      p.lvl2[(size_t(mblk) * p.n_groups + grp) * R + ml] = best;
    }
    if (!arrive_last(p.counters + CNT_MBLK + mblk, p.n_groups, &s_flag)) return;
    if (threadIdx.x < R) {
      const int ml = threadIdx.x;
      unsigned long long best = 0;
      for (int g = 0; g < p.n_groups; ++g) {
        const unsigned long long k = p.lvl2[(size_t(mblk) * p.n_groups + g) * R + ml];
        best = k > best ? k : best;
      }
      const int m = mblk * R + ml;
      if (m < p.M) p.tok_out[m] = key_index(best);
    }
    if (!arrive_last(p.counters + CNT_FINAL, p.m_blocks, &s_flag)) return;
    if (p.verify) {
      const int B = p.block;
      for (int s = threadIdx.x; s < p.batch; s += 256) {
        int L = B;
        for (int j = 0; j < B; ++j) {
          if (p.draft_in[s * B + j] != p.tok_out[s * (B + 1) + j]) { L = j; break; }
        }
        p.accept_len[s] = L;
        p.bonus[s] = p.tok_out[s * (B + 1) + L];
      }
    }
  }
}

template <typename T, int EPI, int NB, int XS>
static hipError_t launch_xs(const GemmParams &p, hipStream_t s) {
  const dim3 grid(p.m_blocks * p.n_blocks * p.splits), block(256);
  switch (p.MT) {
    case 1: hipLaunchKernelGGL((gemm_kernel<T, 1, NB, EPI, XS>), grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL((gemm_kernel<T, 2, NB, EPI, XS>), grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL((gemm_kernel<T, 4, NB, EPI, XS>), grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Activation planes: fp32 storage always has one; bf16 activations that the
// step produces itself carry two (hi + lo), external bf16 inputs one.
template <typename T, int EPI, int NB>
static hipError_t launch_mt(const GemmParams &p, hipStream_t s) {
  if constexpr (Ty<T>::SIZE == 2) {
    if (p.xs == 2) return launch_xs<T, EPI, NB, 2>(p, s);
  }
  return p.xs == 1 ? launch_xs<T, EPI, NB, 1>(p, s) : hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_t(int epi, const GemmParams &p, hipStream_t s) {
  if (epi == EPI_ARGMAX) return p.NB == 2 ? launch_mt<T, EPI_ARGMAX, 2>(p, s) : hipErrorInvalidValue;
  if (p.NB != 4) return hipErrorInvalidValue;
  switch (epi) {
    case EPI_STORE: return launch_mt<T, EPI_STORE, 4>(p, s);
    case EPI_RESID: return launch_mt<T, EPI_RESID, 4>(p, s);
    case EPI_SWIGLU: return launch_mt<T, EPI_SWIGLU, 4>(p, s);
    case EPI_QKV: return launch_mt<T, EPI_QKV, 4>(p, s);
    case EPI_KVINJ: return launch_mt<T, EPI_KVINJ, 4>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm(int dtype, int epi, const GemmParams &p, hipStream_t s) {
  return dtype == DFLASH_BF16 ? launch_t<bf16_t>(epi, p, s) : launch_t<float>(epi, p, s);
}

}  // namespace dflash
