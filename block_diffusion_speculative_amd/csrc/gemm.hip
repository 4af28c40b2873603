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
// whole K range.  Its 16 wavefronts split K, stream their weight tiles
// with non-temporal loads, and add their partial tiles in LDS in a fixed
// order, so the result does not depend on scheduling and no workgroup ever
// waits on another.  The epilogue runs in the same workgroup.  The vocabulary
// argmax is the one cross-workgroup reduction: each workgroup folds its best
// (logit, index) key per row into one of 64 slots with a 64-bit atomic max,
// and a small follow-up kernel reads the slots after the kernel boundary.
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

// Every GEMM workgroup has 16 wavefronts and splits K into the same 16
// contiguous chunks whatever the row-tile count, so a row's result does not
// depend on how many other rows share the launch.
template <int MT> struct GemmShape {
  static constexpr int WAVES = 16;
  static constexpr int THREADS = WAVES * 64;
};

// Largest unroll (power of two, at most 8) whose in-flight fragments plus
// accumulators fit about 25 x 16 bytes per lane (the 128-VGPR budget of a
// 1024-thread workgroup, with room for addresses).
constexpr int pick_unroll(int nb, int mt, int xs) {
  int u = 8;
  while (u > 1 && u * (nb + mt * xs) + mt * nb > 25) u >>= 1;
  return u;
}

template <typename T, int MT, int NB, int EPI, int XS>
__global__ __launch_bounds__(GemmShape<MT>::THREADS) void gemm_kernel(const GemmParams p) {
  constexpr int E = Ty<T>::E, KT = Ty<T>::KT, ES = Ty<T>::SIZE;
  constexpr int WAVES = GemmShape<MT>::WAVES, NT = GemmShape<MT>::THREADS;
  constexpr int U = pick_unroll(NB, MT, XS);  // k-tiles per batch of loads
  constexpr int NF = MT * NB;
  constexpr int R = MT * 16, CN = NB * 16;
  constexpr int ROUND = (32 / NF) < WAVES ? (32 / NF) : WAVES;  // wavefronts per LDS round (<= 32 KiB)
  static_assert(NF * 64 <= NT, "one accumulator element per thread");
  __shared__ f32x4 red[ROUND * NF * 64];

  const int total = p.m_blocks * p.n_blocks;
  const int bid = xcd_remap(blockIdx.x, total);
  const int nblk = bid % p.n_blocks;
  const int mblk = bid / p.n_blocks;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;

  const int nt0 = nblk * NB;
  const int seg = nt0 / p.seg_ntiles;
  const char *wbase = p.w_seg[seg] + size_t(nt0 - seg * p.seg_ntiles) * p.k_tiles * 1024 + lane * 16;
  const size_t wstride = size_t(p.k_tiles) * 1024;

  const int per = (p.k_tiles + WAVES - 1) / WAVES;
  const int k0 = min(wave * per, p.k_tiles);
  const int k1 = min(k0 + per, p.k_tiles);
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
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) wf[u][nb] = ld16_stream(wbase + nb * wstride + size_t(kt + u) * 1024);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int xp = 0; xp < XS; ++xp) xf[u][mt][xp] = load_x(mt, kt + u, xp);
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

  // Sum the wavefronts' partial tiles in wavefront order, ROUND at a time.
  f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
  const int e_own = threadIdx.x;  // element owned in the final tile
  for (int r0 = 0; r0 < WAVES; r0 += ROUND) {
    if (wave >= r0 && wave < r0 + ROUND) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) red[((wave - r0) * NF + mt * NB + nb) * 64 + lane] = acc[mt][nb];
    }
    __syncthreads();
    if (e_own < NF * 64) {
      for (int w = 0; w < ROUND; ++w) {
        if (r0 == 0 && w == 0) sum = red[e_own];
        else sum += red[w * NF * 64 + e_own];
      }
    }
    __syncthreads();
  }
  if (e_own < NF * 64) red[e_own] = sum;
  __syncthreads();

  // ---------------------------------------------------------------- epilogues
  if constexpr (EPI == EPI_STORE || EPI == EPI_RESID) {
    for (int e = threadIdx.x; e < R * CN; e += NT) {
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
    for (int e = threadIdx.x; e < R * HALF * 16; e += NT) {
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
    for (int e = threadIdx.x; e < R * CN; e += NT) {
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
  } else if constexpr (EPI == EPI_ARGMAX) {
    if (threadIdx.x < R) {
      const int ml = threadIdx.x;
      const int m = mblk * R + ml;
      if (m < p.M) {
        unsigned long long best = 0;
        for (int nl = 0; nl < CN; ++nl) {
          const int n = nblk * CN + nl;
          if (n < p.vocab) {
            const unsigned long long k = argmax_key(tile_at(red, NB, ml, nl), n);
            best = k > best ? k : best;
          }
        }
        __hip_atomic_fetch_max(p.keys + size_t(m) * ARGMAX_SLOTS + (nblk % ARGMAX_SLOTS), best,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// Commit the injected rows: ctx_len[s] += n_s unless that exceeds capacity
// (the injection skipped such a sequence and flagged it).
__global__ __launch_bounds__(64) void commit_rows_kernel(int *ctx_len, const int *cu_new, int batch, int capacity) {
  for (int s = threadIdx.x; s < batch; s += blockDim.x) {
    const int ns = cu_new[s + 1] - cu_new[s];
    if (ctx_len[s] + ns <= capacity) ctx_len[s] += ns;
  }
}

template <typename T, int EPI, int NB, int XS>
static hipError_t launch_xs(const GemmParams &p, hipStream_t s) {
  const dim3 grid(p.m_blocks * p.n_blocks);
  switch (p.MT) {
    case 1: hipLaunchKernelGGL((gemm_kernel<T, 1, NB, EPI, XS>), grid, dim3(GemmShape<1>::THREADS), 0, s, p); break;
    case 2: hipLaunchKernelGGL((gemm_kernel<T, 2, NB, EPI, XS>), grid, dim3(GemmShape<2>::THREADS), 0, s, p); break;
    case 4: hipLaunchKernelGGL((gemm_kernel<T, 4, NB, EPI, XS>), grid, dim3(GemmShape<4>::THREADS), 0, s, p); break;
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
  switch (epi) {
    case EPI_STORE: return p.NB == 1 ? launch_mt<T, EPI_STORE, 1>(p, s) : hipErrorInvalidValue;
    case EPI_RESID: return p.NB == 1 ? launch_mt<T, EPI_RESID, 1>(p, s) : hipErrorInvalidValue;
    case EPI_QKV: return p.NB == 1 ? launch_mt<T, EPI_QKV, 1>(p, s) : hipErrorInvalidValue;
    case EPI_KVINJ: return p.NB == 1 ? launch_mt<T, EPI_KVINJ, 1>(p, s) : hipErrorInvalidValue;
    case EPI_SWIGLU: return p.NB == 2 ? launch_mt<T, EPI_SWIGLU, 2>(p, s) : hipErrorInvalidValue;
    case EPI_ARGMAX: return p.NB == 2 ? launch_mt<T, EPI_ARGMAX, 2>(p, s) : hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm(int dtype, int epi, const GemmParams &p, hipStream_t s) {
  return dtype == DFLASH_BF16 ? launch_t<bf16_t>(epi, p, s) : launch_t<float>(epi, p, s);
}

hipError_t launch_argmax_finish(const ArgmaxFinishParams &p, int batch, hipStream_t s) {
  hipLaunchKernelGGL(argmax_finish_kernel, dim3(batch), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_commit_rows(int *ctx_len, const int *cu_new, int batch, int capacity, hipStream_t s) {
  hipLaunchKernelGGL(commit_rows_kernel, dim3(1), dim3(64), 0, s, ctx_len, cu_new, batch, capacity);
  return hipGetLastError();
}

}  // namespace dflash
