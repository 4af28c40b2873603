// Row-wise and data-movement kernels: RMSNorm + pack (with the block
// embedding gather), weight packing, KV-cache layout conversion, fills.
#include "common.hpp"
#include "kernels.hpp"
#include "gemm_util.hpp"

namespace dflash {

// Block embedding, one workgroup per row: slot 0 of a block takes the last
// accepted token, the other slots the mask token.  Writes the fp32 rows, the
// packed rows * gain of the first RMSNorm (rows [M, rows_pad) zeroed) and the
// per-16-column tile sums of squares, in the order tile_ssq16 fixes: a chunk
// of E columns is reduced as a balanced tree in column order and the 16 / E
// chunks of a tile by an xor butterfly.
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const EmbedParams p) {
  constexpr int E = Ty<T>::E, ES = Ty<T>::SIZE;
  constexpr int MAXC = 8;  // chunks per thread: H <= 256 * 8 * E
  const int m = blockIdx.x;
  const int nch = p.H / E;
  if (m >= p.M) {
    for (int c = threadIdx.x; c < nch; c += 256)
      for (int pl = 0; pl < p.planes; ++pl)
        st16(p.xpacked + pl * p.x_plane + packed_offset<T>(m, c * E, p.x_kt), make_uint4(0, 0, 0, 0));
    return;
  }
  const int s = m / p.block, j = m % p.block;
  if (p.anchor_pos && j == 0 && threadIdx.x == 0) {
    int seq = p.anchor_seq[s], pos = p.anchor_pos[s];
    bool bad = seq < 0 || seq >= p.max_batch;
    seq = seq < 0 ? 0 : (seq >= p.max_batch ? p.max_batch - 1 : seq);
    const int have = max(0, min(p.ctx_len[seq], p.capacity));
    bad = bad || pos < 0 || pos > have;
    pos = pos < 0 ? 0 : (pos > have ? have : pos);
    if (bad) atomicOr(p.status, DFLASH_STATUS_ANCHOR);
    p.blk_region[s] = seq;
    p.blk_ctx[s] = pos;
  }
  int tok = p.tokens ? p.tokens[m] : (j == 0 ? p.last_tok[s] : p.mask_id);
  if (tok < 0 || tok >= p.vocab) {
    if (threadIdx.x == 0) atomicOr(p.status, DFLASH_STATUS_TOKEN);
    tok = tok < 0 ? 0 : p.vocab - 1;
  }
  const char *src = p.embed + size_t(tok) * p.H * ES;
#pragma unroll
  for (int k = 0; k < MAXC; ++k) {
    const int c = threadIdx.x + 256 * k;
    if (c < nch) {
      const uint4 v = ld16(src + size_t(c) * 16);
      const uint4 gv = ld16(p.gain + size_t(c) * 16);
      float x[E], sq[E], yh[E], yl[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        x[e] = chunk_get<T>(v, e);
        sq[e] = __fmul_rn(x[e], x[e]);
        split2<T>(x[e] * chunk_get<T>(gv, e), yh[e], yl[e]);
      }
      char *dst = p.xpacked + packed_offset<T>(m, c * E, p.x_kt);
      st16(dst, chunk_pack<T>(yh));
      if (p.planes > 1) st16(dst + p.x_plane, chunk_pack<T>(yl));
      float *gd = p.gathered + size_t(m) * p.H + c * E;
#pragma unroll
      for (int e = 0; e < E; ++e) gd[e] = x[e];
#pragma unroll
      for (int w = 1; w < E; w <<= 1)
#pragma unroll
        for (int e = 0; e < E; e += 2 * w) sq[e] = sq[e] + sq[e + w];
      float t = sq[0];
#pragma unroll
      for (int w = 1; w < 16 / E; w <<= 1) t += __shfl_xor(t, w, 64);
      if ((c & (16 / E - 1)) == 0) p.ssq[size_t(m) * (p.H / 16) + c / (16 / E)] = t;
    }
  }
}

// rs[m] = 1 / sqrt(mean(x_m^2) + eps) from the tile sums (row_rstd8 order).
__global__ __launch_bounds__(256) void rstd_kernel(const float *ssq, int tiles, int K, float eps, int M, float *rs) {
  const int m = blockIdx.x * 32 + (threadIdx.x >> 3);
  if (m >= M) return;  // whole 8-lane groups leave together
  const float v = row_rstd8(ssq + size_t(m) * tiles, tiles, K, eps);
  if ((threadIdx.x & 7) == 0) rs[m] = v;
}

// Pack a row-major [rows, cols] matrix into fragment tiles.  Destination
// row tile rt goes to tile row d = (dst_tile_offset + rt * dst_tile_stride);
// with pairs, row tiles 2p and 2p + 1 interleave per column tile (tile
// (d, c) at position (p * col_tiles + c) * 2 + (d & 1)).  For
// the first rot_rows rows, packed row r of each rot_head_dim-row head takes
// source channel rot_channel(r) of that head (rotary pairs share a tile).
template <typename T>
__global__ __launch_bounds__(256) void pack_matrix_kernel(const char *src, int rows, int cols, char *dst,
                                                          int tile_off, int tile_stride, int rot_hd,
                                                          int rot_rows, bool pairs) {
  constexpr int E = Ty<T>::E, KT = Ty<T>::KT, ES = Ty<T>::SIZE;
  const int ktc = (cols + KT - 1) / KT;
  const int rtc = (rows + 15) / 16;
  const long long total = (long long)rtc * ktc * 64;
  for (long long i = blockIdx.x * 256ll + threadIdx.x; i < total; i += (long long)gridDim.x * 256) {
    const int lane = int(i & 63);
    const long long tile = i >> 6;
    const int ct = int(tile % ktc), rt = int(tile / ktc);
    const int row = rt * 16 + (lane & 15);
    const int col = ct * KT + (lane >> 4) * E;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (row < rows) {
      int srow = row;
      if (row < rot_rows) srow = (row / rot_hd) * rot_hd + rot_channel(row % rot_hd, rot_hd);
      if (col + E <= cols) {
        v = ld16(src + (size_t(srow) * cols + col) * ES);
      } else if (col < cols) {
        float tmp[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          tmp[e] = 0.f;
          if (col + e < cols) {
            const char *sp = src + (size_t(srow) * cols + col + e) * ES;
            if constexpr (ES == 2) tmp[e] = bf16_to_f32(*reinterpret_cast<const uint16_t *>(sp));
            else tmp[e] = *reinterpret_cast<const float *>(sp);
          }
        }
        v = chunk_pack<T>(tmp);
      }
    }
    const long long drt = tile_off + (long long)rt * tile_stride;
    // pairs: row tiles 2p and 2p + 1 interleave per column tile
    const size_t dtile = pairs ? size_t((drt >> 1) * ktc + ct) * 2 + (drt & 1) : size_t(drt) * ktc + ct;
    st16(dst + dtile * 1024 + lane * 16, v);
  }
}

// Plain [regions][capacity][head_dim] <-> packed K / V cache regions.
template <typename T>
__global__ __launch_bounds__(256) void kv_convert_kernel(bool to_packed, char *pk, char *pv, char *k, char *v,
                                                         long long regions, int capacity, int hd) {
  constexpr int ES = Ty<T>::SIZE;
  const long long per_region = (long long)capacity * hd;
  const long long total = regions * per_region;
  for (long long i = blockIdx.x * 256ll + threadIdx.x; i < total; i += (long long)gridDim.x * 256) {
    const long long reg = i / per_region;
    const int rem = int(i % per_region);
    const int pos = rem / hd, dd = rem % hd;
    const size_t rbase = size_t(reg) * per_region * ES;
    char *plain_k = k + size_t(i) * ES, *plain_v = v + size_t(i) * ES;
    char *packed_k = pk + rbase + kcache_offset<T>(pos, dd, hd);
    char *packed_v = pv + rbase + vcache_offset<T>(pos, dd, hd);
    if constexpr (ES == 2) {
      if (to_packed) {
        *reinterpret_cast<uint16_t *>(packed_k) = *reinterpret_cast<const uint16_t *>(plain_k);
        *reinterpret_cast<uint16_t *>(packed_v) = *reinterpret_cast<const uint16_t *>(plain_v);
      } else {
        *reinterpret_cast<uint16_t *>(plain_k) = *reinterpret_cast<const uint16_t *>(packed_k);
        *reinterpret_cast<uint16_t *>(plain_v) = *reinterpret_cast<const uint16_t *>(packed_v);
      }
    } else {
      if (to_packed) {
        *reinterpret_cast<float *>(packed_k) = *reinterpret_cast<const float *>(plain_k);
        *reinterpret_cast<float *>(packed_v) = *reinterpret_cast<const float *>(plain_v);
      } else {
        *reinterpret_cast<float *>(plain_k) = *reinterpret_cast<const float *>(packed_k);
        *reinterpret_cast<float *>(plain_v) = *reinterpret_cast<const float *>(packed_v);
      }
    }
  }
}

__global__ __launch_bounds__(256) void zero_kernel(uint4 *p, size_t n16) {
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < n16; i += size_t(gridDim.x) * 256)
    p[i] = make_uint4(0, 0, 0, 0);
}

static int grid_for(long long work) {
  long long g = (work + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return int(g);
}

hipError_t launch_embed(int dtype, const EmbedParams &p, hipStream_t s) {
  if (dtype == DFLASH_BF16) hipLaunchKernelGGL(embed_kernel<bf16_t>, dim3(p.rows_pad), dim3(256), 0, s, p);
  else hipLaunchKernelGGL(embed_kernel<float>, dim3(p.rows_pad), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_rstd(const float *ssq, int tiles, int K, float eps, int M, float *rs, hipStream_t s) {
  hipLaunchKernelGGL(rstd_kernel, dim3((M + 31) / 32), dim3(256), 0, s, ssq, tiles, K, eps, M, rs);
  return hipGetLastError();
}

hipError_t launch_pack_matrix(int dtype, const void *src, int rows, int cols, void *dst, int tile_off,
                              int tile_stride, int rot_hd, int rot_rows, bool pairs, hipStream_t s) {
  const int kt = kt_of(dtype);
  const long long work = (long long)((rows + 15) / 16) * ((cols + kt - 1) / kt) * 64;
  if (dtype == DFLASH_BF16)
    hipLaunchKernelGGL(pack_matrix_kernel<bf16_t>, dim3(grid_for(work)), dim3(256), 0, s,
                       (const char *)src, rows, cols, (char *)dst, tile_off, tile_stride, rot_hd, rot_rows, pairs);
  else
    hipLaunchKernelGGL(pack_matrix_kernel<float>, dim3(grid_for(work)), dim3(256), 0, s,
                       (const char *)src, rows, cols, (char *)dst, tile_off, tile_stride, rot_hd, rot_rows, pairs);
  return hipGetLastError();
}

hipError_t launch_kv_convert(int dtype, bool to_packed, void *pk, void *pv, void *k, void *v,
                             long long regions, int capacity, int hd, hipStream_t s) {
  const long long work = regions * capacity * hd;
  if (dtype == DFLASH_BF16)
    hipLaunchKernelGGL(kv_convert_kernel<bf16_t>, dim3(grid_for(work)), dim3(256), 0, s, to_packed,
                       (char *)pk, (char *)pv, (char *)k, (char *)v, regions, capacity, hd);
  else
    hipLaunchKernelGGL(kv_convert_kernel<float>, dim3(grid_for(work)), dim3(256), 0, s, to_packed,
                       (char *)pk, (char *)pv, (char *)k, (char *)v, regions, capacity, hd);
  return hipGetLastError();
}

// One workgroup per row: out = x / sqrt(mean(x^2) + eps) * gain in the
// storage type (the target's final normalised hidden state, the verify
// head's input); the sum of squares runs per thread in order and then over a
// fixed tree.
template <typename T>
__global__ __launch_bounds__(256) void rownorm_kernel(const float *x, int H, const T *gain, float eps, char *out) {
  __shared__ float red[256];
  const float *r = x + size_t(blockIdx.x) * H;
  float s = 0.f;
  for (int c = threadIdx.x; c < H; c += 256) s += __fmul_rn(r[c], r[c]);
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (int(threadIdx.x) < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const float inv = 1.0f / sqrtf(red[0] / float(H) + eps);
  for (int c = threadIdx.x; c < H; c += 256)
    store_elem<T>(out + (size_t(blockIdx.x) * H + c) * Ty<T>::SIZE, r[c] * inv * to_f32<T>(gain[c]));
}

__global__ void kv_commit_kernel(int *ctx_len, const int *accept_len, int batch, int max_commit, int capacity) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= batch) return;
  const int add = min(max(accept_len[s] + 1, 0), max_commit);
  ctx_len[s] = min(ctx_len[s] + add, capacity);
}

hipError_t launch_rownorm(int dtype, const float *x, int M, int H, const void *gain, float eps, void *out,
                          hipStream_t s) {
  if (dtype == DFLASH_BF16)
    hipLaunchKernelGGL(rownorm_kernel<bf16_t>, dim3(M), dim3(256), 0, s, x, H,
                       static_cast<const bf16_t *>(gain), eps, static_cast<char *>(out));
  else
    hipLaunchKernelGGL(rownorm_kernel<float>, dim3(M), dim3(256), 0, s, x, H, static_cast<const float *>(gain),
                       eps, static_cast<char *>(out));
  return hipGetLastError();
}

hipError_t launch_kv_commit(int *ctx_len, const int *accept_len, int batch, int max_commit, int capacity,
                            hipStream_t s) {
  hipLaunchKernelGGL(kv_commit_kernel, dim3((batch + 63) / 64), dim3(64), 0, s, ctx_len, accept_len, batch,
                     max_commit, capacity);
  return hipGetLastError();
}

hipError_t launch_zero(void *p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3(grid_for((long long)n16)), dim3(256), 0, s, (uint4 *)p, n16);
  return hipGetLastError();
}

}  // namespace dflash
