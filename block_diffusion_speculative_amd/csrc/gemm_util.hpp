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
__device__ inline float rope_apply(float v, float partner, int dd, int d, int pos, const GemmParams &p) {
  if (!p.rope_on) return v;
  const int half = d >> 1;
  const double t = double(pos) * p.rope_turns[dd % half];
  const float f = float(t - floor(t));
  const float c = __builtin_amdgcn_cosf(f), s = __builtin_amdgcn_sinf(f);
  return dd < half ? v * c - partner * s : v * c + partner * s;
}

template <typename T> __device__ inline void store_elem(char *p, float v);
template <> __device__ inline void store_elem<float>(char *p, float v) { *reinterpret_cast<float *>(p) = v; }
template <> __device__ inline void store_elem<bf16_t>(char *p, float v) {
  *reinterpret_cast<uint16_t *>(p) = f32_to_bf16(v);
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
