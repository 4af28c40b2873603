// Device helpers shared by the GEMM kernels: rotary embedding on one
// element, element stores, the orderable argmax key and the last-arriver
// handshake.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace dflash {

// Rotate-half RoPE on one element.  The angle pos * theta^(-2i/d) is formed
// in turns (host-computed theta^(-2i/d) / 2pi in fp64), reduced to [0, 1) in
// fp64, and fed to the hardware sin/cos, which take turns.
// turns: theta^(-2i/d) / 2pi of the element's pair i = dd mod d/2.
__device__ inline float rope_rotate(float v, float partner, int dd, int d, int pos, double turns) {
  const double t = double(pos) * turns;
  const float f = float(t - floor(t));
  const float c = __builtin_amdgcn_cosf(f), s = __builtin_amdgcn_sinf(f);
  return dd < (d >> 1) ? v * c - partner * s : v * c + partner * s;
}
__device__ inline float rope_apply(float v, float partner, int dd, int d, int pos, const GemmParams &p) {
  if (!p.rope_on) return v;
  return rope_rotate(v, partner, dd, d, pos, p.rope_turns[dd % (d >> 1)]);
}

template <typename T> __device__ inline void store_elem(char *p, float v);
template <> __device__ inline void store_elem<float>(char *p, float v) { *reinterpret_cast<float *>(p) = v; }
template <> __device__ inline void store_elem<bf16_t>(char *p, float v) {
  *reinterpret_cast<uint16_t *>(p) = f32_to_bf16(v);
}

// Four consecutive elements of one row (col0 a multiple of 4: one lane chunk
// of a packed tile) in a single 8-byte (bf16) or 16-byte (fp32) store.
template <typename T> __device__ inline void store_elem4(char *p, const f32x4 &v);
template <> __device__ inline void store_elem4<float>(char *p, const f32x4 &v) { *reinterpret_cast<f32x4 *>(p) = v; }
template <> __device__ inline void store_elem4<bf16_t>(char *p, const f32x4 &v) {
  *reinterpret_cast<uint2 *>(p) = make_uint2(f32x2_to_bf16x2(v[0], v[1]), f32x2_to_bf16x2(v[2], v[3]));
}

// A causal pass's new K (is_k) or V element of sequence s, KV head g,
// channel dd (the packed rotary order for K) at cache position pos of layer
// layer0; a position past the capacity sets DFLASH_STATUS_CAPACITY instead.
template <typename T>
__device__ inline void qkv_cache_store(const GemmParams &p, bool is_k, int s, int g, int pos, int dd, float v) {
  if (pos >= p.capacity) {
    if (dd == 0) atomicOr(p.status, DFLASH_STATUS_CAPACITY);
    return;
  }
  const int d = p.head_dim;
  const size_t region = size_t(p.capacity) * d * Ty<T>::SIZE;
  char *base = (is_k ? p.kcache : p.vcache) + ((size_t(p.layer0) * p.max_batch + s) * p.n_kv + g) * region;
  store_elem<T>(base + (is_k ? kcache_offset<T>(pos, dd, d) : vcache_offset<T>(pos, dd, d)), v);
}

// Store four consecutive columns col0 .. col0 + 3 (col0 a multiple of 4) of
// one row into a packed activation buffer: they sit in one lane chunk, so
// each plane takes a single 8-byte (bf16) or 16-byte (fp32) store.
template <typename T> __device__ inline void store_split4(char *p, size_t plane_bytes, int planes, const f32x4 &v);
template <> __device__ inline void store_split4<float>(char *p, size_t, int, const f32x4 &v) {
  *reinterpret_cast<f32x4 *>(p) = v;
}
template <> __device__ inline void store_split4<bf16_t>(char *p, size_t plane_bytes, int planes, const f32x4 &v) {
  const uint32_t h01 = f32x2_to_bf16x2(v[0], v[1]), h23 = f32x2_to_bf16x2(v[2], v[3]);
  *reinterpret_cast<uint2 *>(p) = make_uint2(h01, h23);
  if (planes > 1) {
    const uint32_t l01 = f32x2_to_bf16x2(v[0] - __uint_as_float(h01 << 16), v[1] - __uint_as_float(h01 & 0xffff0000u));
    const uint32_t l23 = f32x2_to_bf16x2(v[2] - __uint_as_float(h23 << 16), v[3] - __uint_as_float(h23 & 0xffff0000u));
    *reinterpret_cast<uint2 *>(p + plane_bytes) = make_uint2(l01, l23);
  }
}

// The same for four consecutive K channels dd0 .. dd0 + 3 (dd0 a multiple
// of 4 in the packed rotary order) of one position.
template <typename T>
__device__ inline void qkv_cache_store_k4(const GemmParams &p, int s, int g, int pos, int dd0, const f32x4 &v) {
  if (pos >= p.capacity) {
    if (dd0 == 0) atomicOr(p.status, DFLASH_STATUS_CAPACITY);
    return;
  }
  const int d = p.head_dim;
  const size_t region = size_t(p.capacity) * d * Ty<T>::SIZE;
  char *base = p.kcache + ((size_t(p.layer0) * p.max_batch + s) * p.n_kv + g) * region;
  store_elem4<T>(base + kcache_offset<T>(pos, dd0, d), v);
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

// 16-byte accesses with the cache policy the compiler gives agent-scope
// atomic loads and stores (sc1): the partial tiles of a split item pass
// between workgroups that may sit on different XCDs, whose L2s are not
// coherent with each other.  The ordering comes from the handshake below:
// a writer's stores are complete (vmcnt(0)) before its arrival is counted,
// and a reader issues its loads only after the count has told it that every
// writer arrived.
constexpr int CPOL_AGENT = 16;
__device__ inline void st16_agent(__amdgpu_buffer_rsrc_t r, int voff, int soff, const f32x4 &v) {
  const u32x4 u = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
  __builtin_amdgcn_raw_buffer_store_b128(u, r, voff, soff, CPOL_AGENT);
}
__device__ inline f32x4 ld16_agent(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, CPOL_AGENT);
  return f32x4{__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w)};
}

// True in every thread of the workgroup that arrives last.  Each wavefront
// first waits for all of its vector-memory operations (so its atomics and
// stores are performed), the workgroup synchronises, and one thread counts
// the arrival with a device-scope atomic.
__device__ inline bool last_arriver(unsigned *arrive, int *flag) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0)
    *flag = __hip_atomic_fetch_add(arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1;
  __syncthreads();
  return *flag != 0;
}

// The same for a count of `total` arrivals at *counter (any workgroups).
__device__ inline bool last_arriver_of(unsigned *counter, unsigned total, int *flag) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0)
    *flag = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == total - 1;
  __syncthreads();
  return *flag != 0;
}

}  // namespace dflash
