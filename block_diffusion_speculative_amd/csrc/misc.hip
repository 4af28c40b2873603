// Row-wise and data-movement kernels: RMSNorm + pack (with the block
// embedding gather), weight packing, KV-cache layout conversion, fills.
#include "common.hpp"
#include "kernels.hpp"

namespace dflash {

// One workgroup per row.  Embedding mode gathers the block's token row
// (slot 0: the last accepted token, other slots: the mask token) and keeps an
// fp32 copy; then y = x / sqrt(mean(x^2) + eps) * gain is written as packed
// fragment tiles (and optionally as fp32).  Rows in [M, rows_pad) are zeroed.
template <typename T>
__global__ __launch_bounds__(256) void norm_pack_kernel(const NormParams p) {
  constexpr int E = Ty<T>::E, ES = Ty<T>::SIZE;
  constexpr int MAXC = 8;  // chunks per thread: H <= 256 * 8 * E
  __shared__ float red[4];
  const int m = blockIdx.x;
  const int nch = p.H / E;
  if (m >= p.M) {
    for (int c = threadIdx.x; c < nch; c += 256)
      for (int pl = 0; pl < p.planes; ++pl)
        st16(p.xpacked + pl * p.x_plane + packed_offset<T>(m, c * E, p.x_kt), make_uint4(0, 0, 0, 0));
    return;
  }
  const char *src_t = nullptr;
  if (p.embed) {
    const int s = m / p.block, j = m % p.block;
    int tok = j == 0 ? p.last_tok[s] : p.mask_id;
    if (tok < 0 || tok >= p.vocab) {
      if (threadIdx.x == 0) atomicOr(p.status, DFLASH_STATUS_TOKEN);
      tok = tok < 0 ? 0 : p.vocab - 1;
    }
    src_t = p.embed + size_t(tok) * p.H * ES;
  }
  float x[MAXC][E];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < MAXC; ++k) {
    const int c = threadIdx.x + 256 * k;
    if (c < nch) {
      if (src_t) {
        const uint4 v = ld16(src_t + size_t(c) * 16);
#pragma unroll
        for (int e = 0; e < E; ++e) x[k][e] = chunk_get<T>(v, e);
      } else {
        const float *r = p.src + size_t(m) * p.H + c * E;
#pragma unroll
        for (int e = 0; e < E; ++e) x[k][e] = r[e];
      }
#pragma unroll
      for (int e = 0; e < E; ++e) ss += x[k][e] * x[k][e];
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = ((red[0] + red[1]) + red[2]) + red[3];
  const float r = 1.0f / sqrtf(tot / float(p.H) + p.eps);
#pragma unroll
  for (int k = 0; k < MAXC; ++k) {
    const int c = threadIdx.x + 256 * k;
    if (c < nch) {
      const uint4 gv = ld16(p.gain + size_t(c) * 16);
      float y[E], yh[E], yl[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        y[e] = x[k][e] * r * chunk_get<T>(gv, e);
        split2<T>(y[e], yh[e], yl[e]);
      }
      char *dst = p.xpacked + packed_offset<T>(m, c * E, p.x_kt);
      st16(dst, chunk_pack<T>(yh));
      if (p.planes > 1) st16(dst + p.x_plane, chunk_pack<T>(yl));
      if (p.gathered) {
        float *gd = p.gathered + size_t(m) * p.H + c * E;
#pragma unroll
        for (int e = 0; e < E; ++e) gd[e] = x[k][e];
      }
      if (p.normed) {
        float *nd = p.normed + size_t(m) * p.H + c * E;
#pragma unroll
        for (int e = 0; e < E; ++e) nd[e] = y[e];
      }
    }
  }
}

// Pack a row-major [rows, cols] matrix into fragment tiles.  Destination
// row tile rt goes to tile row (dst_tile_offset + rt * dst_tile_stride).  For
// the first rot_rows rows, packed row r of each rot_head_dim-row head takes
// source channel rot_channel(r) of that head (rotary pairs share a tile).
template <typename T>
__global__ __launch_bounds__(256) void pack_matrix_kernel(const char *src, int rows, int cols, char *dst,
                                                          int tile_off, int tile_stride, int rot_hd,
                                                          int rot_rows) {
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
    const size_t dtile = size_t(tile_off + (long long)rt * tile_stride) * ktc + ct;
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

hipError_t launch_norm_pack(int dtype, const NormParams &p, hipStream_t s) {
  if (dtype == DFLASH_BF16)
    hipLaunchKernelGGL(norm_pack_kernel<bf16_t>, dim3(p.rows_pad), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(norm_pack_kernel<float>, dim3(p.rows_pad), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_pack_matrix(int dtype, const void *src, int rows, int cols, void *dst, int tile_off,
                              int tile_stride, int rot_hd, int rot_rows, hipStream_t s) {
  const int kt = kt_of(dtype);
  const long long work = (long long)((rows + 15) / 16) * ((cols + kt - 1) / kt) * 64;
  if (dtype == DFLASH_BF16)
    hipLaunchKernelGGL(pack_matrix_kernel<bf16_t>, dim3(grid_for(work)), dim3(256), 0, s,
                       (const char *)src, rows, cols, (char *)dst, tile_off, tile_stride, rot_hd, rot_rows);
  else
    hipLaunchKernelGGL(pack_matrix_kernel<float>, dim3(grid_for(work)), dim3(256), 0, s,
                       (const char *)src, rows, cols, (char *)dst, tile_off, tile_stride, rot_hd, rot_rows);
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

hipError_t launch_zero(void *p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_kernel, dim3(grid_for((long long)n16)), dim3(256), 0, s, (uint4 *)p, n16);
  return hipGetLastError();
}

}  // namespace dflash
