// Block attention of the drafting pass: every block query attends to all
// cached (injected) context positions and to every block slot, with no mask
// ("DFlash, Diffusion LLMs, dLLM, MTP and Speculative Decoding: A Deep
// Research Report", "Why DFlash beats EAGLE-3" item 3; "Term: DFlash
// speculative decoding", "DFlash: architecture and workflow").
//
// One workgroup per (sequence, KV head, context split); its wavefronts are the
// query heads of that KV head's group, so each K/V step is read from HBM once
// and staged in LDS for the whole group.  A step is KT positions (32 for
// bf16): S^T = K Q^T on MFMA gives each lane 4 positions x 1 query per
// 16-position tile, the online softmax runs in registers with row statistics
// exchanged by lane shuffles, and O^T += V^T P^T consumes the probabilities
// straight from the S^T registers (the V cache layout stores positions in
// that register order).  Each split writes (O, running max, running sum) and
// a merge kernel combines the splits with a log-sum-exp weighting.
#include "common.hpp"
#include "kernels.hpp"

namespace dflash {

template <typename T> __device__ inline float round_to(float v);
template <> __device__ inline float round_to<float>(float v) { return v; }
template <> __device__ inline float round_to<bf16_t>(float v) { return bf16_to_f32(f32_to_bf16(v)); }

// Zero the elements of a V chunk whose positions are >= nvalid.
template <typename T> __device__ inline uint4 mask_v_chunk(uint4 v, int g, int nvalid);
template <> __device__ inline uint4 mask_v_chunk<float>(uint4 v, int g, int nvalid) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (4 * g + e >= nvalid) w[e] = 0;
  return make_uint4(w[0], w[1], w[2], w[3]);
}
template <> __device__ inline uint4 mask_v_chunk<bf16_t>(uint4 v, int g, int nvalid) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int pos = 16 * (e >> 2) + 4 * g + (e & 3);
    if (pos >= nvalid) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <typename T, int HD, int XS>
__global__ __launch_bounds__(1024) void attn_kernel(const AttnParams p) {
  constexpr int KT = Ty<T>::KT, ES = Ty<T>::SIZE;
  constexpr int DT = HD / KT, DV = HD / 16, KTT = KT / 16;
  constexpr int KB = KTT * DT * 1024, VB = DV * 1024;
  constexpr int REC = DV * 256 + 32;
  __shared__ uint4 lds[(KB + VB) / 16];

  const int z = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = g * p.group + wave;
  const int C = min(p.ctx_len[s], p.capacity);
  const int n_ctx = (C + KT - 1) / KT;
  const int total = n_ctx + 1;
  const int per = (total + p.splits - 1) / p.splits;
  const int st0 = min(z * per, total), st1 = min(st0 + per, total);

  uint4 qf[XS][DT];
  {
    const char *qb = p.qbuf + (size_t(s) * p.n_q + h) * DT * 1024;
    const bool ok = (lane & 15) < p.block;
#pragma unroll
    for (int xp = 0; xp < XS; ++xp)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        qf[xp][dt] = ok ? ld16(qb + xp * p.q_plane + dt * 1024 + lane * 16) : make_uint4(0, 0, 0, 0);
  }
  float m_run = -1e30f, l_run = 0.f;
  f32x4 o[DV];
#pragma unroll
  for (int i = 0; i < DV; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const size_t region = size_t(p.capacity) * HD * ES;
  const char *kreg = p.kcache + (size_t(s) * p.n_kv + g) * region;
  const char *vreg = p.vcache + (size_t(s) * p.n_kv + g) * region;
  const char *kbk = p.kblk + (size_t(s) * p.n_kv + g) * KB;
  const char *vbk = p.vblk + (size_t(s) * p.n_kv + g) * VB;
  const int gq = lane >> 4;

  for (int st = st0; st < st1; ++st) {
    const bool blk = st == n_ctx;
    const char *ksrc = blk ? kbk : kreg + size_t(st) * KB;
    const char *vsrc = blk ? vbk : vreg + size_t(st) * VB;
    const int nvalid = blk ? p.block : min(KT, C - st * KT);
    __syncthreads();
    for (int c = threadIdx.x; c < (KB + VB) / 16; c += blockDim.x) {
      uint4 v;
      if (c < KB / 16) {
        v = ld16(ksrc + size_t(c) * 16);
      } else {
        const int cv = c - KB / 16;
        v = ld16(vsrc + size_t(cv) * 16);
        if (nvalid < KT) v = mask_v_chunk<T>(v, (cv & 63) >> 4, nvalid);
      }
      lds[c] = v;
    }
    __syncthreads();

    f32x4 sacc[KTT];
#pragma unroll
    for (int t = 0; t < KTT; ++t) {
      sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int xp = 0; xp < XS; ++xp) sacc[t] = mma<T>(sacc[t], lds[(t * DT + dt) * 64 + lane], qf[xp][dt]);
    }
    float sv[KTT * 4];
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < KTT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pos = 16 * t + 4 * gq + i;
        const float x = pos < nvalid ? sacc[t][i] * p.scale_log2 : -INFINITY;
        sv[4 * t + i] = x;
        mx = fmaxf(mx, x);
      }
    mx = warp_max_xor(mx, 16);
    mx = warp_max_xor(mx, 32);
    const float m_new = fmaxf(m_run, mx);
    const float corr = exp2f(m_run - m_new);
    // Probabilities: with XS == 2 they enter the MFMA as hi + lo planes and
    // the row sum uses the fp32 values; with XS == 1 both use the rounded ones.
    float ph[KTT * 4], pl[KTT * 4];
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < KTT * 4; ++e) {
      const float pr = exp2f(sv[e] - m_new);
      if constexpr (XS == 2) {
        split2<T>(pr, ph[e], pl[e]);
        ps += pr;
      } else {
        ph[e] = round_to<T>(pr);
        ps += ph[e];
      }
    }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    l_run = l_run * corr + ps;
    const uint4 pf = chunk_pack<T>(ph);
    uint4 pfl = make_uint4(0, 0, 0, 0);
    if constexpr (XS == 2) pfl = chunk_pack<T>(pl);
#pragma unroll
    for (int dv = 0; dv < DV; ++dv) {
      o[dv] *= corr;
      const uint4 vf = lds[KB / 16 + dv * 64 + lane];
      o[dv] = mma<T>(o[dv], vf, pf);
      if constexpr (XS == 2) o[dv] = mma<T>(o[dv], vf, pfl);
    }
    m_run = m_new;
  }

  float *rec = p.part + ((size_t(s) * p.n_q + h) * p.splits + z) * REC;
#pragma unroll
  for (int dv = 0; dv < DV; ++dv) reinterpret_cast<f32x4 *>(rec)[dv * 64 + lane] = o[dv];
  if (lane < 16) {
    rec[DV * 256 + lane] = m_run;
    rec[DV * 256 + 16 + lane] = l_run;
  }
}

// Combine the splits of one (sequence, query head, 16-channel tile).
template <typename T, int HD>
__global__ __launch_bounds__(64) void attn_merge_kernel(const AttnParams p) {
  constexpr int DV = HD / 16;
  constexpr int REC = DV * 256 + 32;
  const int dv = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int lane = threadIdx.x, q = lane & 15;
  const float *base = p.part + (size_t(s) * p.n_q + h) * p.splits * REC;
  float M = -1e30f;
  for (int z = 0; z < p.splits; ++z) M = fmaxf(M, base[size_t(z) * REC + DV * 256 + q]);
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  for (int z = 0; z < p.splits; ++z) {
    const float *r = base + size_t(z) * REC;
    const float w = exp2f(r[DV * 256 + q] - M);
    L += w * r[DV * 256 + 16 + q];
    const f32x4 ov = reinterpret_cast<const f32x4 *>(r)[dv * 64 + lane];
    acc += w * ov;
  }
  if (q >= p.block) return;
  const float inv = 1.0f / L;
  const int row = s * p.block + q;
  const int nqd = p.n_q * HD;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int col = h * HD + dv * 16 + 4 * (lane >> 4) + i;
    const float v = acc[i] * inv;
    p.attn_out[size_t(row) * nqd + col] = v;
    store_split<T>(p.xo + packed_offset<T>(row, col, p.xo_kt), p.xo_plane, p.xs, v);
  }
}

template <typename T, int XS>
static hipError_t launch_attn_xs(const AttnParams &p, int batch, hipStream_t s) {
  const dim3 grid(p.splits, p.n_kv, batch), block(64 * p.group);
  if (p.head_dim == 128) hipLaunchKernelGGL((attn_kernel<T, 128, XS>), grid, block, 0, s, p);
  else if (p.head_dim == 64) hipLaunchKernelGGL((attn_kernel<T, 64, XS>), grid, block, 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_attn_t(const AttnParams &p, int batch, hipStream_t s) {
  if constexpr (Ty<T>::SIZE == 2) {
    if (p.xs == 2) return launch_attn_xs<T, 2>(p, batch, s);
  }
  return p.xs == 1 ? launch_attn_xs<T, 1>(p, batch, s) : hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_merge_t(const AttnParams &p, int batch, hipStream_t s) {
  const dim3 grid(p.head_dim / 16, p.n_q, batch), block(64);
  if (p.head_dim == 128) hipLaunchKernelGGL((attn_merge_kernel<T, 128>), grid, block, 0, s, p);
  else if (p.head_dim == 64) hipLaunchKernelGGL((attn_merge_kernel<T, 64>), grid, block, 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_attention(int dtype, const AttnParams &p, int batch, hipStream_t s) {
  return dtype == DFLASH_BF16 ? launch_attn_t<bf16_t>(p, batch, s) : launch_attn_t<float>(p, batch, s);
}

hipError_t launch_attn_merge(int dtype, const AttnParams &p, int batch, hipStream_t s) {
  return dtype == DFLASH_BF16 ? launch_merge_t<bf16_t>(p, batch, s) : launch_merge_t<float>(p, batch, s);
}

}  // namespace dflash
