// Temperature sampling: drafted tokens sampled from the drafter's
// distribution, and speculative-sampling verification against the
// target's.  ("Term: DFlash speculative decoding", "DFlash: architecture and
// workflow": the speculator fills the masked positions with sampled tokens,
// and the target checks each drafted token against its argmax or an
// acceptance criterion; "DFlash, Diffusion LLMs, dLLM, MTP and Speculative
// Decoding: A Deep Research Report", "DFlash benchmark results": results at
// temperature 1.)
//
// At temperature T the drafter's distribution at slot j is
// q_j = softmax(l_j / T) and the target's p_j = softmax(l'_j / T).  The
// criterion is the standard speculative-sampling rule: drafted token d_j is
// accepted with probability min(1, p_j(d_j) / q_j(d_j)), in slot order; at
// the first rejected slot j the next token is drawn from the normalised
// residual max(0, p_j - q_j), and when all B slots are accepted from p_B.
// Random numbers come in as uniforms in (0, 1); a categorical draw is the
// Gumbel-max: the lowest-index argmax over the vocabulary of
// log w(v) - log(-log u(v)).  The logit rows live in HBM (the heads store
// them instead of folding an argmax); every kernel here streams them once.
#include "common.hpp"
#include "kernels.hpp"
#include "gemm_util.hpp"

namespace dflash {

constexpr int SAMPLE_THREADS = 256;

// Gumbel noise -log(-log u).  -log u is taken as -log1p(u - 1) above 1/2,
// where u - 1 is exact, so a u close to 1 keeps its precision; u is clamped
// into (0, 1) (the largest float below 1 gives about 16.6).
__device__ inline float gumbel_of(float u) {
  u = fminf(fmaxf(u, 1e-37f), 0x1.fffffep-1f);
  const float t = u < 0.5f ? -logf(u) : -log1pf(u - 1.0f);
  return -logf(t);
}

// Largest key over the workgroup (a 64-lane shuffle max, then LDS); every
// thread gets the result.
__device__ inline unsigned long long block_max_key(unsigned long long k) {
  __shared__ unsigned long long part[SAMPLE_THREADS / 64];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const unsigned long long o = __shfl_xor(k, off, 64);
    k = o > k ? o : k;
  }
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = k;
  __syncthreads();
  k = part[0];
#pragma unroll
  for (int w = 1; w < SAMPLE_THREADS / 64; ++w) k = part[w] > k ? part[w] : k;
  __syncthreads();
  return k;
}

// One chunk of one row's vocabulary: the row's best key over the chunk goes
// to its argmax slot (chunk), folded later by argmax_finish_kernel.
__global__ __launch_bounds__(SAMPLE_THREADS) void gumbel_draft_kernel(const SampleParams p) {
  const int m = blockIdx.y, chunk = blockIdx.x;
  const int per = (p.vocab + p.chunks - 1) / p.chunks;
  const int v0 = chunk * per, v1 = min(v0 + per, p.vocab);
  const float *lg = p.logits + size_t(m) * p.ld;
  const float *u = p.u + size_t(m) * p.vocab;
  unsigned long long best = 0;
  for (int v = v0 + threadIdx.x; v < v1; v += SAMPLE_THREADS) {
    const unsigned long long k = argmax_key(lg[v] * p.inv_t + gumbel_of(u[v]), v);
    best = k > best ? k : best;
  }
  best = block_max_key(best);
  if (threadIdx.x == 0 && best != 0)
    __hip_atomic_fetch_max(p.keys + size_t(m) * ARGMAX_SLOTS + chunk, best, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// log sum_v exp(l(v) * inv_t) of a row, in two launches.  Every chunk of
// the row keeps a running (max, sum of exp(x - max)) per thread over its
// strided elements in order (rescaling the sum when the max grows), the
// threads are merged by a fixed tree, and the chunk's pair goes to part;
// row_lse_merge_kernel then merges a row's chunk pairs in chunk order.  The
// result is deterministic.
__device__ inline void lse_merge(float &m, float &s, float m2, float s2) {
  const float mm = fmaxf(m, m2);
  if (mm == -INFINITY) return;   // both empty
  s = s * expf(m - mm) + s2 * expf(m2 - mm);
  m = mm;
}

__global__ __launch_bounds__(SAMPLE_THREADS) void row_lse_part_kernel(const float *logits, int ld, int vocab,
                                                                       float inv_t, int chunks, float2 *part) {
  __shared__ float rm[SAMPLE_THREADS], rsum[SAMPLE_THREADS];
  const int row = blockIdx.y, chunk = blockIdx.x;
  const float *lg = logits + size_t(row) * ld;
  const int per = (vocab + chunks - 1) / chunks;
  const int v0 = chunk * per, v1 = min(v0 + per, vocab);
  float m = -INFINITY, sum = 0.f;
  for (int v = v0 + threadIdx.x; v < v1; v += SAMPLE_THREADS) {
    const float x = lg[v] * inv_t;
    if (x > m) {
      sum = sum * expf(m - x) + 1.0f;
      m = x;
    } else {
      sum += expf(x - m);
    }
  }
  rm[threadIdx.x] = m;
  rsum[threadIdx.x] = sum;
  __syncthreads();
  for (int w = SAMPLE_THREADS / 2; w >= 1; w >>= 1) {
    if (int(threadIdx.x) < w) {
      float a = rm[threadIdx.x], b = rsum[threadIdx.x];
      lse_merge(a, b, rm[threadIdx.x + w], rsum[threadIdx.x + w]);
      rm[threadIdx.x] = a;
      rsum[threadIdx.x] = b;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) part[size_t(row) * chunks + chunk] = make_float2(rm[0], rsum[0]);
}

__global__ __launch_bounds__(64) void row_lse_merge_kernel(const float2 *part, int chunks, int rows, float *lse) {
  const int row = blockIdx.x * 64 + threadIdx.x;
  if (row >= rows) return;
  float m = -INFINITY, sum = 0.f;
  for (int c = 0; c < chunks; ++c) {
    const float2 pc = part[size_t(row) * chunks + c];
    lse_merge(m, sum, pc.x, pc.y);
  }
  lse[row] = m + logf(sum);
}

// One chunk of one sequence's vocabulary.  Every workgroup of the sequence
// first replays the acceptance scan (16 slots at most, so each finds the
// same first rejected slot j); chunk 0 stores the accepted length.  Then the
// chunk's candidates for the next token: the residual max(0, p_j - q_j)
// when a slot was rejected (candidates with no residual mass are never
// picked over one that has some), else p_B.
__global__ __launch_bounds__(SAMPLE_THREADS) void spec_sample_kernel(const SampleParams p) {
  __shared__ int js;
  const int s = blockIdx.y, chunk = blockIdx.x, B = p.block;
  if (threadIdx.x == 0) {
    int j = 0;
    for (; j < B; ++j) {
      const int d = min(max(p.draft[s * B + j], 0), p.vocab - 1);
      const int rq = s * B + j, rp = s * (B + 1) + j;
      const float logq = p.q_logits[size_t(rq) * p.ld + d] * p.inv_t - p.lse_q[rq];
      const float logp = p.p_logits[size_t(rp) * p.ld + d] * p.inv_t - p.lse_p[rp];
      // accept with probability min(1, p / q): u <= p / q
      if (!(logf(p.u_accept[s * B + j]) <= logp - logq)) break;
    }
    js = j;
    if (chunk == 0) p.accept_len[s] = j;
  }
  __syncthreads();
  const int j = js;
  const int rp = s * (B + 1) + j;
  const float *lp = p.p_logits + size_t(rp) * p.ld;
  const float *u = p.u_resid + size_t(s) * p.vocab;
  const int per = (p.vocab + p.chunks - 1) / p.chunks;
  const int v0 = chunk * per, v1 = min(v0 + per, p.vocab);
  unsigned long long best = 0;
  if (j < B) {
    const int rq = s * B + j;
    const float *lq = p.q_logits + size_t(rq) * p.ld;
    const float lsp = p.lse_p[rp], lsq = p.lse_q[rq];
    for (int v = v0 + threadIdx.x; v < v1; v += SAMPLE_THREADS) {
      const float w = expf(lp[v] * p.inv_t - lsp) - expf(lq[v] * p.inv_t - lsq);
      const float val = w > 0.f ? logf(w) + gumbel_of(u[v]) : -INFINITY;
      const unsigned long long k = argmax_key(val, v);
      best = k > best ? k : best;
    }
  } else {
    for (int v = v0 + threadIdx.x; v < v1; v += SAMPLE_THREADS) {
      const unsigned long long k = argmax_key(lp[v] * p.inv_t + gumbel_of(u[v]), v);
      best = k > best ? k : best;
    }
  }
  best = block_max_key(best);
  if (threadIdx.x == 0 && best != 0)
    __hip_atomic_fetch_max(p.keys + size_t(s) * ARGMAX_SLOTS + chunk, best, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_gumbel_draft(const SampleParams &p, int rows, hipStream_t s) {
  if (p.chunks < 1 || p.chunks > ARGMAX_SLOTS) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gumbel_draft_kernel, dim3(p.chunks, rows), dim3(SAMPLE_THREADS), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_row_lse(const float *logits, int ld, int vocab, float inv_t, int rows, int chunks, float2 *part,
                          float *lse, hipStream_t s) {
  if (chunks < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(row_lse_part_kernel, dim3(chunks, rows), dim3(SAMPLE_THREADS), 0, s, logits, ld, vocab, inv_t,
                     chunks, part);
  hipLaunchKernelGGL(row_lse_merge_kernel, dim3((rows + 63) / 64), dim3(64), 0, s, part, chunks, rows, lse);
  return hipGetLastError();
}

hipError_t launch_spec_sample(const SampleParams &p, int batch, hipStream_t s) {
  if (p.chunks < 1 || p.chunks > ARGMAX_SLOTS) return hipErrorInvalidValue;
  hipLaunchKernelGGL(spec_sample_kernel, dim3(p.chunks, batch), dim3(SAMPLE_THREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace dflash
