// Device-side building blocks shared by the gfx950 kernels: element types,
// bf16 rounding, the 16x16 MFMA step on packed fragment tiles, layout index
// math and the cross-workgroup "last arriver" handshake.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dflash.h"

namespace dflash {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Storage type tags.  bf16 values are carried as raw uint16 bit patterns.
struct bf16_t { uint16_t bits; };

template <typename T> struct Ty;
template <> struct Ty<float> {
  static constexpr int E = 4;     // elements per 16-byte lane chunk
  static constexpr int KT = 16;   // columns per fragment tile
  static constexpr int SIZE = 4;
};
template <> struct Ty<bf16_t> {
  static constexpr int E = 8;
  static constexpr int KT = 32;
  static constexpr int SIZE = 2;
};

__host__ __device__ inline int kt_of(int dtype) { return dtype == DFLASH_BF16 ? 32 : 16; }
__host__ __device__ inline int esize_of(int dtype) { return dtype == DFLASH_BF16 ? 2 : 4; }

__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Round to nearest even with the hardware conversion (v_cvt_pk_bf16_f32).
__device__ inline uint32_t f32x2_to_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}
__device__ inline uint16_t f32_to_bf16(float f) { return uint16_t(f32x2_to_bf16x2(f, 0.f)); }

template <typename T> __device__ inline float to_f32(T v);
template <> __device__ inline float to_f32<float>(float v) { return v; }
template <> __device__ inline float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v.bits); }

template <typename T> __device__ inline T from_f32(float v);
template <> __device__ inline float from_f32<float>(float v) { return v; }
template <> __device__ inline bf16_t from_f32<bf16_t>(float v) { return bf16_t{f32_to_bf16(v)}; }

// Element e (0 <= e < E) of a 16-byte chunk, as fp32.
template <typename T> __device__ inline float chunk_get(const uint4 &c, int e);
template <> __device__ inline float chunk_get<float>(const uint4 &c, int e) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  return __uint_as_float(w[e]);
}
template <> __device__ inline float chunk_get<bf16_t>(const uint4 &c, int e) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  return bf16_to_f32(uint16_t(w[e >> 1] >> ((e & 1) * 16)));
}

// Build a 16-byte chunk from E fp32 values (rounded to T).
template <typename T> __device__ inline uint4 chunk_pack(const float *v);
template <> __device__ inline uint4 chunk_pack<float>(const float *v) {
  return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                    __float_as_uint(v[3]));
}
template <> __device__ inline uint4 chunk_pack<bf16_t>(const float *v) {
  return make_uint4(f32x2_to_bf16x2(v[0], v[1]), f32x2_to_bf16x2(v[2], v[3]), f32x2_to_bf16x2(v[4], v[5]),
                    f32x2_to_bf16x2(v[6], v[7]));
}

// Split x into hi + lo parts of T (hi = T(x), lo = T(x - hi)); for fp32
// storage lo is zero.  Two bf16 planes carry ~16 mantissa bits.
template <typename T> __device__ inline void split2(float x, float &hi, float &lo);
template <> __device__ inline void split2<float>(float x, float &hi, float &lo) { hi = x; lo = 0.f; }
template <> __device__ inline void split2<bf16_t>(float x, float &hi, float &lo) {
  hi = bf16_to_f32(f32_to_bf16(x));
  lo = x - hi;
}

// Store one element into plane 0 (and its remainder into plane 1 when
// planes == 2) of a packed activation buffer.
template <typename T> __device__ inline void store_split(char *p, size_t plane_bytes, int planes, float v);
template <> __device__ inline void store_split<float>(char *p, size_t, int, float v) {
  *reinterpret_cast<float *>(p) = v;
}
template <> __device__ inline void store_split<bf16_t>(char *p, size_t plane_bytes, int planes, float v) {
  const uint16_t h = f32_to_bf16(v);
  *reinterpret_cast<uint16_t *>(p) = h;
  if (planes > 1) *reinterpret_cast<uint16_t *>(p + plane_bytes) = f32_to_bf16(v - bf16_to_f32(h));
}

// acc += A * B for one pair of packed fragment chunks.  A's lane (r, g)
// holds row r of A, B's lane (r, g) holds column r of B; both carry the same
// E contraction indices, so the product contracts over 4E indices.  Result
// lane (c, g) holds rows 4g..4g+3 of column c.
template <typename T> __device__ inline f32x4 mma(f32x4 acc, const uint4 &a, const uint4 &b);
template <> __device__ inline f32x4 mma<bf16_t>(f32x4 acc, const uint4 &a, const uint4 &b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
template <> __device__ inline f32x4 mma<float>(f32x4 acc, const uint4 &a, const uint4 &b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  return acc;
}

__device__ inline uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ inline void st16(void *p, const uint4 &v) { *reinterpret_cast<uint4 *>(p) = v; }
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
// Streaming load for data read exactly once (weights): non-temporal hint.
__device__ inline uint4 ld16_stream(const void *p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Raw buffer resource word 3 for gfx9-family parts (32-bit data format), and
// a 16-byte streaming (non-temporal) load through a buffer resource: byte
// voff (per lane) + soff (uniform) from the resource base.
constexpr int BUF_DWORD3 = 0x00020000;
// A pointer every lane holds the same value of, moved to scalar registers so
// that a buffer resource built from it needs no per-lane loop.
__device__ inline const char *uniform_ptr(const char *p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v)), hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return reinterpret_cast<const char *>((uint64_t(hi) << 32) | lo);
}
__device__ inline uint4 ld16_buf_stream(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2 /* nt */);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// ------------------------------------------------------------------ layouts

// Byte offset of element (row, col) in a packed matrix whose rows hold
// kt_count column tiles.
template <typename T>
__host__ __device__ inline size_t packed_offset(int row, int col, int kt_count) {
  constexpr int E = Ty<T>::E, KT = Ty<T>::KT;
  const size_t tile = size_t(row >> 4) * kt_count + col / KT;
  const int lane = (row & 15) + 16 * ((col % KT) / E);
  return tile * 1024 + lane * 16 + (col % E) * Ty<T>::SIZE;
}

// K cache region of one (layer, sequence, kv head): positions in 16-row
// tiles, head_dim in KT-column tiles (the A operand of S^T = K Q^T).
template <typename T>
__host__ __device__ inline size_t kcache_offset(int pos, int dd, int head_dim) {
  return packed_offset<T>(pos, dd, head_dim / Ty<T>::KT);
}

// V cache region: one KT-position step holds head_dim/16 tiles; tile lane
// (r, g) holds channel r and the E positions 16*(e/4) + 4g + (e%4), which is
// the order in which the S^T accumulators of that step hold the positions
// (the A operand of O^T = V^T P^T).
template <typename T>
__host__ __device__ inline size_t vcache_offset(int pos, int dd, int head_dim) {
  constexpr int KT = Ty<T>::KT;
  const int step = pos / KT, kk = pos % KT;
  const int t = kk >> 4, rem = kk & 15;
  const int g = rem >> 2, e = 4 * t + (rem & 3);
  const size_t tile = size_t(step) * (head_dim / 16) + (dd >> 4);
  return tile * 1024 + ((dd & 15) + 16 * g) * 16 + e * Ty<T>::SIZE;
}

// Rotary pairs: packed row r of a q/k head holds channel
// rot_channel(r) so that channels i and i + d/2 sit in rows r and r ^ 8.
__host__ __device__ inline int rot_channel(int r, int head_dim) {
  const int t = r >> 4, p = r & 15;
  return p < 8 ? 8 * t + p : head_dim / 2 + 8 * t + (p - 8);
}

// ------------------------------------------------------------- RMSNorm

// The RMSNorm statistics are assembled from per-(row, 16-column tile) sums of
// squares.  A tile's sum is the balanced binary tree over its 16 squares in
// column order (what an xor butterfly over 16 lanes computes).  A row's total
// takes its tiles in 8 contiguous runs of 4 * ceil(tiles / 32) (the last runs
// may be short or empty): run q is summed in order by lane q of an 8-lane
// group, and the runs are combined by an xor butterfly.  Every kernel that
// forms these values uses this order, so they agree bit for bit.
constexpr int RSTD_MAX_TILES = 512;  // hidden <= 8192

__device__ inline float tile_ssq16(float v) {
  float s = __fmul_rn(v, v);  // rounded square: never contracted into the adds
  s += __shfl_xor(s, 1, 64);
  s += __shfl_xor(s, 2, 64);
  s += __shfl_xor(s, 4, 64);
  s += __shfl_xor(s, 8, 64);
  return s;
}

// 1 / sqrt(mean(x^2) + eps) of one row from its tile sums (tiles a multiple
// of 4, 16-byte aligned); called by the 8 lanes (8-aligned) of a group, lane
// q = lane & 7; every lane gets the result.  Loads go out 8 at a time.
__device__ inline float row_rstd8(const float *tile_ssq, int tiles, int K, float eps) {
  constexpr int V = 8;  // 16-byte loads per pass
  const int q = threadIdx.x & 7;
  const int run = 4 * ((tiles + 31) / 32);
  const int t0 = min(q * run, tiles), t1 = min(t0 + run, tiles);
  float s = 0.f;
  for (int base = t0; base < t0 + run; base += 4 * V) {
    f32x4 v[V];
#pragma unroll
    for (int i = 0; i < V; ++i) v[i] = *reinterpret_cast<const f32x4 *>(tile_ssq + min(base + 4 * i, tiles - 4));
#pragma unroll
    for (int i = 0; i < V; ++i) {
      if (base + 4 * i < t1) {
        s += v[i][0];
        s += v[i][1];
        s += v[i][2];
        s += v[i][3];
      }
    }
  }
  s += __shfl_xor(s, 1, 64);
  s += __shfl_xor(s, 2, 64);
  s += __shfl_xor(s, 4, 64);
  return 1.0f / sqrtf(s / float(K) + eps);
}

// Direct global -> LDS load (global_load_lds_dwordx4): lane l's 16 bytes
// from src land at lds_base + 16 l, lds_base uniform over the wavefront (M0
// holds its LDS byte address).  Issued as inline assembly so that the
// compiler does not wait for every such load before each LDS read; callers
// wait with wait_vmcnt (the loads count in vmcnt) and an LDS barrier.
__device__ inline void load_lds16(const void *src, void *lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(lds_base)));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(src) : "memory", "m0");
}

// The same with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane
// byte offset (the instruction's scalar-base form): no 64-bit address per
// lane has to stay live between loads.
__device__ inline void load_lds16_s(const char *sbase, uint32_t voff, const void *lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(lds_base)));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

// Wait until at most N of this wavefront's vector-memory operations are
// outstanding (direct-to-LDS loads included); other counters untouched.
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Barrier for LDS traffic only: waits for this wavefront's LDS operations,
// not for its outstanding global loads (which __syncthreads would drain).
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ------------------------------------------------------------- dispatch

// Workgroups of one launch are dispatched round-robin over the 8 XCDs; remap
// so that consecutive logical ids share an XCD (and its L2).
__device__ inline int xcd_remap(int bid, int nblocks) {
  if (nblocks % 8 != 0) return bid;
  return (bid % 8) * (nblocks / 8) + bid / 8;
}

__device__ inline float warp_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}

}  // namespace dflash
