// Block attention of the drafting pass: every block query attends to all
// cached (injected) context positions and to every block slot, with no mask
// ("DFlash, Diffusion LLMs, dLLM, MTP and Speculative Decoding: A Deep
// Research Report", "Why DFlash beats EAGLE-3" item 3; "Term: DFlash
// speculative decoding", "DFlash: architecture and workflow").
//
// One workgroup per (sequence, KV head, share of its query heads, context
// split).  Its wavefronts are the workgroup's query heads times SUB
// sub-splits (at most 16 wavefronts).  A step is KT positions (32 for bf16);
// round r stages the SUB steps st0 + r * SUB + ss in LDS, where wavefront
// (head, ss) takes step ss.  The K/V tiles go straight from global memory to
// LDS (global_load_lds_dwordx4, 1 KiB per wavefront instruction), two rounds
// in flight, so a short split (the batch-1 case) has all of its loads out at
// once.  Per step: S^T = K Q^T on MFMA gives each lane 4 positions x 1 query
// per 16-position tile, the online softmax runs in registers with row
// statistics exchanged by lane shuffles, and O^T += V^T P^T consumes the
// probabilities straight from the S^T registers (the V cache layout stores
// positions in that register order).  q enters as hi + lo planes when XS ==
// 2, and so does P for bf16 (two MFMAs per V tile: a single bf16 plane of P
// adds about 0.1% to every layer's attention output, which compounds over
// the layers).  The sub-splits are then merged in LDS with log-sum-exp
// weights, every wavefront taking a slice of its head's channels; a single
// split writes the output itself, several write (O, running max, running
// sum) records that attn_merge_kernel combines.
#include "common.hpp"
#include "kernels.hpp"
#include "gemm_util.hpp"

namespace dflash {

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

constexpr int ATTN_MAX_WAVES = 16;
constexpr int ATTN_MAX_SUB = 4;
constexpr int ATTN_MAX_SPLITS = 32;

// Sub-splits per workgroup holding `heads` query heads.
__host__ __device__ inline int attn_sub(int heads) {
  const int s = ATTN_MAX_WAVES / heads;
  return s < 1 ? 1 : (s > ATTN_MAX_SUB ? ATTN_MAX_SUB : s);
}

// RC: 1 KiB tiles each wavefront loads per round (a compile-time count, so the
// wait for the older of two rounds in flight is an immediate).  NW: most
// wavefronts per workgroup (8 leaves each 256 VGPRs, 16 leaves 128).
// MASK: a causal or tree pass (block positions masked per query row).
template <typename T, int HD, int XS, int RC, int NW, bool MASK>
__global__ __launch_bounds__(NW * 64) void attn_kernel(const AttnParams p) {
  constexpr int KT = Ty<T>::KT, ES = Ty<T>::SIZE;
  constexpr int DT = HD / KT, DV = HD / 16, KTT = KT / 16;
  constexpr int KB = KTT * DT * 1024, VB = DV * 1024, SB = KB + VB;
  constexpr int TPS = SB / 1024;                    // tiles per step
  constexpr int REC = DV * 256 + 32;                // floats of one merge record
  constexpr int RING = 2 * ATTN_MAX_SUB * SB / 16;  // uint4 of two rounds
  constexpr int MREC = ATTN_MAX_WAVES * REC / 4;    // uint4 of one record per wavefront
  __shared__ uint4 lds[RING > MREC ? RING : MREC];

  const int z = blockIdx.x;
  const int QT = p.q_tiles, qt = blockIdx.z % QT;   // query tile
  int s = blockIdx.z / QT;                           // sequence
  if (p.sort_seqs) {
    // Workgroups are dispatched in grid order with the sequence slowest, so
    // taking the sequences by rank (longest context first, ties by index)
    // starts the longest work first when the grid needs more than one wave
    // of workgroups.
    __shared__ int ctx_s[MAX_SEQS], seq_of_rank[MAX_SEQS];
    const int nseq = int(gridDim.z) / QT;
    if (int(threadIdx.x) < nseq) ctx_s[threadIdx.x] = min(p.ctx_len[threadIdx.x], p.capacity);
    __syncthreads();
    if (int(threadIdx.x) < nseq) {
      const int t = threadIdx.x, lt = ctx_s[t];
      int rank = 0;
      for (int u = 0; u < nseq; ++u) rank += ctx_s[u] > lt || (ctx_s[u] == lt && u < t);
      seq_of_rank[rank] = t;
    }
    __syncthreads();
    s = seq_of_rank[s];
  }
  const int g = blockIdx.y / p.head_split, hs = blockIdx.y % p.head_split;
  const int gw = p.group / p.head_split;            // query heads of this workgroup
  const int waves = blockDim.x >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int SUB = attn_sub(gw);
  const int hl = wave % gw, ss = wave / gw;
  const int h = g * p.group + hs * gw + hl;
  const int C = min(p.ctx_len[s], p.capacity);
  const int n_ctx = (C + KT - 1) / KT;
  const int total = n_ctx + 1;
  const int per = (total + p.splits - 1) / p.splits;
  const int st0 = min(z * per, total), st1 = min(st0 + per, total);
  const int rounds = (st1 - st0 + SUB - 1) / SUB;
  const int round_tiles = SUB * TPS;

  const size_t region = size_t(p.capacity) * HD * ES;
  const int cs = p.region_of ? p.region_of[s] : s;   // the cached sequence this block reads
  const char *kreg = p.kcache + (size_t(cs) * p.n_kv + g) * region;
  const char *vreg = p.vcache + (size_t(cs) * p.n_kv + g) * region;
  const char *kbk = p.kblk + (size_t(s) * p.n_kv + g) * KB;
  const char *vbk = p.vblk + (size_t(s) * p.n_kv + g) * VB;

  // Round r goes to ring slot r % 2.  Wavefront w loads tiles w, w + waves, ...
  // of the round; a tile past the round or of a step past st1 reloads a valid
  // tile into its own slot position (never read), so every wavefront issues
  // exactly RC loads.
  auto issue_round = [&](int r) {
    uint4 *slot = lds + (r & 1) * (ATTN_MAX_SUB * SB / 16);
#pragma unroll
    for (int i = 0; i < RC; ++i) {
      int j = wave + i * waves;
      j = j < round_tiles ? j : round_tiles - 1;
      const int st = st0 + r * SUB + j / TPS, tt = j % TPS;
      const char *src;
      if (st >= st1) src = kbk;
      else if (tt < KB / 1024) src = (st == n_ctx ? kbk : kreg + size_t(st) * KB) + tt * 1024;
      else src = (st == n_ctx ? vbk : vreg + size_t(st) * VB) + (tt - KB / 1024) * 1024;
      load_lds16_s(src, lane * 16, slot + j * 64);
    }
  };

  uint4 qf[XS][DT];
  {
    const char *qb = p.qbuf + ((size_t(s) * p.n_q + h) * QT + qt) * DT * 1024;
    const bool ok = qt * 16 + (lane & 15) < p.block;
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
  const int gq = lane >> 4;
  // Which of this lane's block-step positions its query row sees: all valid
  // slots, or under a causal pass those at or before the row, or under a
  // tree pass the row's ancestors and itself (row_mask bits).  Bit 4t + i
  // stands for position 16t + 4gq + i, as in the S^T accumulators.
  unsigned blk_seen = 0;
  if constexpr (MASK) {
    const int qrow = qt * 16 + (lane & 15);
    const unsigned anc = p.row_mask ? (qrow < p.block ? p.row_mask[s * p.block + qrow] : 0u) : ~0u;
#pragma unroll
    for (int t = 0; t < KTT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pos = 16 * t + 4 * gq + i;
        const bool ok = pos < p.block && !(p.causal && pos > qrow) && ((anc >> pos) & 1u);
        blk_seen |= unsigned(ok) << (4 * t + i);
      }
  }

  auto compute = [&](int st, const uint4 *kl) {
    const bool blk = st == n_ctx;
    const int nvalid = blk ? p.block : min(KT, C - st * KT);
    const uint4 *vl = kl + KB / 16;
    f32x4 sacc[KTT];
#pragma unroll
    for (int t = 0; t < KTT; ++t) {
      sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int xp = 0; xp < XS; ++xp) sacc[t] = mma<T>(sacc[t], kl[(t * DT + dt) * 64 + lane], qf[xp][dt]);
    }
    float sv[KTT * 4];
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < KTT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pos = 16 * t + 4 * gq + i;
        bool seen = pos < nvalid;
        if constexpr (MASK) seen = blk ? ((blk_seen >> (4 * t + i)) & 1u) != 0 : seen;
        const float x = seen ? sacc[t][i] * p.scale_log2 : -INFINITY;
        sv[4 * t + i] = x;
        mx = fmaxf(mx, x);
      }
    mx = warp_max_xor(mx, 16);
    mx = warp_max_xor(mx, 32);
    const float m_new = fmaxf(m_run, mx);
    const float corr = exp2f(m_run - m_new);
    // Probabilities as hi + lo planes of T (about 16 mantissa bits for bf16;
    // fp32 needs one); the row sum takes the fp32 values.
    float ph[KTT * 4], pl[KTT * 4];
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < KTT * 4; ++e) {
      const float pe = exp2f(sv[e] - m_new);
      split2<T>(pe, ph[e], pl[e]);
      ps += pe;
    }
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    l_run = l_run * corr + ps;
    const uint4 pf = chunk_pack<T>(ph);
    const uint4 pfl = chunk_pack<T>(pl);
#pragma unroll
    for (int dv = 0; dv < DV; ++dv) {
      o[dv] *= corr;
      uint4 vf = vl[dv * 64 + lane];
      // positions past nvalid hold stale data: zero them (P is 0 there, but
      // 0 * NaN would not be)
      if (nvalid < KT) vf = mask_v_chunk<T>(vf, gq, nvalid);
      o[dv] = mma<T>(o[dv], vf, pf);
      if constexpr (Ty<T>::SIZE == 2) o[dv] = mma<T>(o[dv], vf, pfl);
    }
    m_run = m_new;
  };

  if (rounds > 0) issue_round(0);
  if (rounds > 1) issue_round(1);
  for (int r = 0; r < rounds; ++r) {
    if (r + 1 < rounds) wait_vmcnt<RC>();
    else wait_vmcnt<0>();
    lds_barrier();
    const int st = st0 + r * SUB + ss;
    if (st < st1) compute(st, lds + (r & 1) * (ATTN_MAX_SUB * SB / 16) + ss * (SB / 16));
    lds_barrier();
    if (r + 2 < rounds) issue_round(r + 2);
  }

  // Merge the sub-splits: every wavefront leaves its record in LDS, then
  // wavefront (head, ss) combines channel tiles ss, ss + SUB, ... of its head
  // over the SUB records (log-sum-exp weights) and writes them out.
  float *recs = reinterpret_cast<float *>(lds);
  {
    float *mine = recs + size_t(wave) * REC;
#pragma unroll
    for (int dv = 0; dv < DV; ++dv) reinterpret_cast<f32x4 *>(mine)[dv * 64 + lane] = o[dv];
    if (lane < 16) {
      mine[DV * 256 + lane] = m_run;
      mine[DV * 256 + 16 + lane] = l_run;
    }
  }
  lds_barrier();
  const int q = lane & 15;
  float M = -1e30f;
  for (int j = 0; j < SUB; ++j) M = fmaxf(M, recs[size_t(j * gw + hl) * REC + DV * 256 + q]);
  float L = 0.f;
  for (int j = 0; j < SUB; ++j) {
    const float *r = recs + size_t(j * gw + hl) * REC;
    L += exp2f(r[DV * 256 + q] - M) * r[DV * 256 + 16 + q];
  }
  const bool final_out = p.splits == 1;
  const float inv = 1.0f / L;
  float *rec = p.part + (((size_t(s) * QT + qt) * p.n_q + h) * p.splits + z) * REC;
  for (int dv = ss; dv < DV; dv += SUB) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < SUB; ++j) {
      const float *r = recs + size_t(j * gw + hl) * REC;
      acc += exp2f(r[DV * 256 + q] - M) * reinterpret_cast<const f32x4 *>(r)[dv * 64 + lane];
    }
    if (final_out) {
      if (qt * 16 + q < p.block) {
        // four consecutive channels: one 16-byte and one packed store
        const int row = s * p.block + qt * 16 + q;
        const int col = h * HD + dv * 16 + 4 * (lane >> 4);
        const f32x4 v = acc * inv;
        *reinterpret_cast<f32x4 *>(p.attn_out + size_t(row) * (p.n_q * HD) + col) = v;
        store_split4<T>(p.xo + packed_offset<T>(row, col, p.xo_kt), p.xo_plane, p.xs, v);
      }
    } else {
      reinterpret_cast<f32x4 *>(rec)[dv * 64 + lane] = acc;
    }
  }
  if (!final_out && ss == 0 && lane < 16) {
    rec[DV * 256 + lane] = M;
    rec[DV * 256 + 16 + lane] = L;
  }
}

// Combine the splits of one (sequence, query head, 16-channel tile): lane
// takes one O^T chunk of every split; all loads are issued before any is used.
template <typename T, int HD, int ZMAX>
__global__ __launch_bounds__(64) void attn_merge_kernel(const AttnParams p) {
  constexpr int DV = HD / 16;
  constexpr int REC = DV * 256 + 32;
  const int dv = blockIdx.x, h = blockIdx.y;
  const int QT = p.q_tiles, s = blockIdx.z / QT, qt = blockIdx.z % QT;
  const int lane = threadIdx.x, q = lane & 15;
  const float *base = p.part + ((size_t(s) * QT + qt) * p.n_q + h) * p.splits * REC;
  float mz[ZMAX], lz[ZMAX];
  f32x4 oz[ZMAX];
#pragma unroll
  for (int z = 0; z < ZMAX; ++z) {
    const float *r = base + size_t(min(z, p.splits - 1)) * REC;
    mz[z] = r[DV * 256 + q];
    lz[z] = r[DV * 256 + 16 + q];
    oz[z] = reinterpret_cast<const f32x4 *>(r)[dv * 64 + lane];
  }
  float M = -1e30f;
#pragma unroll
  for (int z = 0; z < ZMAX; ++z)
    if (z < p.splits) M = fmaxf(M, mz[z]);
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
#pragma unroll
  for (int z = 0; z < ZMAX; ++z) {
    if (z < p.splits) {
      const float w = exp2f(mz[z] - M);
      L += w * lz[z];
      acc += w * oz[z];
    }
  }
  if (qt * 16 + q >= p.block) return;
  // four consecutive channels: one 16-byte and one packed store
  const int row = s * p.block + qt * 16 + q;
  const int col = h * HD + dv * 16 + 4 * (lane >> 4);
  const f32x4 v = acc * (1.0f / L);
  *reinterpret_cast<f32x4 *>(p.attn_out + size_t(row) * (p.n_q * HD) + col) = v;
  store_split4<T>(p.xo + packed_offset<T>(row, col, p.xo_kt), p.xo_plane, p.xs, v);
}

template <typename T, int HD, int XS, int NW, bool MASK>
static hipError_t launch_attn_mask(const AttnParams &p, int batch, int rc, int threads, hipStream_t s) {
  const dim3 grid(p.splits, p.n_kv * p.head_split, batch * p.q_tiles), block(threads);
  if (rc <= 2) hipLaunchKernelGGL((attn_kernel<T, HD, XS, 2, NW, MASK>), grid, block, 0, s, p);
  else if (rc <= 4) hipLaunchKernelGGL((attn_kernel<T, HD, XS, 4, NW, MASK>), grid, block, 0, s, p);
  else if (rc <= 8) hipLaunchKernelGGL((attn_kernel<T, HD, XS, 8, NW, MASK>), grid, block, 0, s, p);
  else if (rc <= 16) hipLaunchKernelGGL((attn_kernel<T, HD, XS, 16, NW, MASK>), grid, block, 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename T, int HD, int XS, int NW>
static hipError_t launch_attn_nw(const AttnParams &p, int batch, int rc, int threads, hipStream_t s) {
  if (p.causal || p.row_mask) return launch_attn_mask<T, HD, XS, NW, true>(p, batch, rc, threads, s);
  return launch_attn_mask<T, HD, XS, NW, false>(p, batch, rc, threads, s);
}

template <typename T, int HD, int XS>
static hipError_t launch_attn_rc(const AttnParams &p, int batch, hipStream_t s) {
  constexpr int SB = (Ty<T>::KT / 16) * (HD / Ty<T>::KT) * 1024 + (HD / 16) * 1024;
  const int sub = attn_sub(p.group / p.head_split);
  const int waves = p.group / p.head_split * sub;
  const int threads = 64 * waves;
  const int rc = (sub * (SB / 1024) + waves - 1) / waves;  // tiles per wavefront per round
  if (waves <= 8) return launch_attn_nw<T, HD, XS, 8>(p, batch, rc, threads, s);
  return launch_attn_nw<T, HD, XS, 16>(p, batch, rc, threads, s);
}

template <typename T, int XS>
static hipError_t launch_attn_xs(const AttnParams &p, int batch, hipStream_t s) {
  if (p.group < 1 || p.group > ATTN_MAX_WAVES || p.splits < 1 || p.splits > ATTN_MAX_SPLITS) return hipErrorInvalidValue;
  if (p.head_split < 1 || p.group % p.head_split) return hipErrorInvalidValue;
  if (p.q_tiles < 1 || p.block > 16 * p.q_tiles || p.block > Ty<T>::KT) return hipErrorInvalidValue;
  if (p.head_dim == 128) return launch_attn_rc<T, 128, XS>(p, batch, s);
  if (p.head_dim == 64) return launch_attn_rc<T, 64, XS>(p, batch, s);
  return hipErrorInvalidValue;
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
  const dim3 grid(p.head_dim / 16, p.n_q, batch * p.q_tiles), block(64);
  if (p.q_tiles < 1) return hipErrorInvalidValue;
  if (p.splits > ATTN_MAX_SPLITS) return hipErrorInvalidValue;
  if (p.head_dim == 128) {
    if (p.splits <= 2) hipLaunchKernelGGL((attn_merge_kernel<T, 128, 2>), grid, block, 0, s, p);
    else if (p.splits <= 16) hipLaunchKernelGGL((attn_merge_kernel<T, 128, 16>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((attn_merge_kernel<T, 128, ATTN_MAX_SPLITS>), grid, block, 0, s, p);
  } else if (p.head_dim == 64) {
    if (p.splits <= 2) hipLaunchKernelGGL((attn_merge_kernel<T, 64, 2>), grid, block, 0, s, p);
    else if (p.splits <= 16) hipLaunchKernelGGL((attn_merge_kernel<T, 64, 16>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((attn_merge_kernel<T, 64, ATTN_MAX_SPLITS>), grid, block, 0, s, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attention(int dtype, const AttnParams &p, int batch, hipStream_t s) {
  return dtype == DFLASH_BF16 ? launch_attn_t<bf16_t>(p, batch, s) : launch_attn_t<float>(p, batch, s);
}

hipError_t launch_attn_merge(int dtype, const AttnParams &p, int batch, hipStream_t s) {
  return dtype == DFLASH_BF16 ? launch_merge_t<bf16_t>(p, batch, s) : launch_merge_t<float>(p, batch, s);
}

}  // namespace dflash
