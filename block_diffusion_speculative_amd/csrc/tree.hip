// Draft trees ("LLMs hit ludicrous speed: diffusion decoding and dMoE
// supercharge AI inference, shattering old benchmarks", the DDTree
// paragraph: continuations built best-first from per-position
// distributions, verified in one target pass under an ancestor-only
// attention mask).
//
// The drafter's block pass gives every slot j a distribution q_j; a
// continuation t_1 .. t_k scores sum_j log q_j(t_j), and the tree holds the
// N best continuations over the top-K tokens of each slot (a prefix scores
// at least as much as its extensions, so they form a tree).  The build pops
// continuations in score order from a heap, pushing after each pop the next
// sibling and the first child of the popped node; verification runs the
// target over the N + 1 nodes (node i at position ctx + depth(i), seeing its
// ancestors), the walk follows the target's argmax down the tree, and the
// accepted path's K/V rows are moved into place in the target cache.
#include "common.hpp"
#include "kernels.hpp"
#include "gemm_util.hpp"

namespace dflash {

constexpr int TREE_MAX_K = 8;
constexpr int TREE_MAX_NODES = 32;   // N + 1 rows of one target pass
constexpr int TOPK_THREADS = 256;

// Top-K keys per row (64-bit (logit, index) keys: larger logit first, then
// lower index), in two launches so that a row's vocabulary is read by many
// workgroups: row_topk_part_kernel takes the K best keys of each of
// TOPK_CHUNKS vocabulary chunks of a row, row_topk_merge_kernel the K best of
// a row's TOPK_CHUNKS * K chunk keys.  Keys are unique, so the result is the
// row's exact top-K in key order.
// K rounds of a workgroup max over the threads' sorted key lists (each
// thread's keys in best[0 .. K), best first; 0 marks no key): round r
// writes the r-th best key of the workgroup to out[r] (thread 0).
__device__ inline void wg_extract_topk(const unsigned long long (&best)[TREE_MAX_K], int K, unsigned long long *out,
                                       unsigned long long *part, int *owner_sh) {
  int head = 0;   // this thread's next unextracted key
  for (int r = 0; r < K; ++r) {
    unsigned long long mine = 0;
#pragma unroll
    for (int i = 0; i < TREE_MAX_K; ++i)
      if (i == head && i < K) mine = best[i];
    unsigned long long k = mine;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const unsigned long long o = __shfl_xor(k, off, 64);
      k = o > k ? o : k;
    }
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = k;
    __syncthreads();
    k = part[0];
#pragma unroll
    for (int w = 1; w < TOPK_THREADS / 64; ++w) k = part[w] > k ? part[w] : k;
    if (k != 0 && mine == k) *owner_sh = threadIdx.x;
    __syncthreads();
    if (int(threadIdx.x) == *owner_sh && k != 0) ++head;
    if (threadIdx.x == 0) out[r] = k;
    __syncthreads();
  }
}

__device__ inline void topk_insert(unsigned long long (&best)[TREE_MAX_K], int K, unsigned long long k) {
#pragma unroll
  for (int i = 0; i < TREE_MAX_K; ++i) {   // insertion into a sorted list
    if (i < K && k > best[i]) {
      const unsigned long long t = best[i];
      best[i] = k;
      k = t;
    }
  }
}

__global__ __launch_bounds__(TOPK_THREADS) void row_topk_part_kernel(const float *logits, int ld, int vocab, int K,
                                                                      unsigned long long *chunk_keys) {
  __shared__ unsigned long long part[TOPK_THREADS / 64];
  __shared__ unsigned long long out[TREE_MAX_K];
  __shared__ int owner_sh;
  const int c = blockIdx.x, row = blockIdx.y;
  const int len = (vocab + TOPK_CHUNKS - 1) / TOPK_CHUNKS;
  const int v0 = c * len, v1 = min(v0 + len, vocab);
  const float *lg = logits + size_t(row) * ld;
  unsigned long long best[TREE_MAX_K];
#pragma unroll
  for (int i = 0; i < TREE_MAX_K; ++i) best[i] = 0;
  for (int v = v0 + int(threadIdx.x); v < v1; v += TOPK_THREADS) topk_insert(best, K, argmax_key(lg[v], v));
  wg_extract_topk(best, K, out, part, &owner_sh);
  if (int(threadIdx.x) < K) chunk_keys[(size_t(row) * TOPK_CHUNKS + c) * K + threadIdx.x] = out[threadIdx.x];
}

__global__ __launch_bounds__(TOPK_THREADS) void row_topk_merge_kernel(const float *logits, int ld, int vocab, int K,
                                                                       const unsigned long long *chunk_keys,
                                                                       const float *lse, float *topk_val,
                                                                       int *topk_idx) {
  __shared__ unsigned long long part[TOPK_THREADS / 64];
  __shared__ unsigned long long out[TREE_MAX_K];
  __shared__ int owner_sh;
  const int row = blockIdx.x;
  unsigned long long best[TREE_MAX_K];
#pragma unroll
  for (int i = 0; i < TREE_MAX_K; ++i) best[i] = 0;
  for (int i = threadIdx.x; i < TOPK_CHUNKS * K; i += TOPK_THREADS)
    topk_insert(best, K, chunk_keys[size_t(row) * TOPK_CHUNKS * K + i]);
  wg_extract_topk(best, K, out, part, &owner_sh);
  if (int(threadIdx.x) < K) {
    // K <= vocab, so every round extracts a real key
    const int idx = min(max(key_index(out[threadIdx.x]), 0), vocab - 1);
    topk_idx[row * K + threadIdx.x] = idx;
    topk_val[row * K + threadIdx.x] = logits[size_t(row) * ld + idx] - lse[row];
  }
}

// One thread per sequence: the best-first heap over (score, depth, rank,
// parent node); ties go to the smaller depth, then to the smaller rank.
// Each thread's heap and node scores live in LDS (a private array indexed
// at run time would live in scratch memory).
constexpr int TREE_THREADS = 64;
struct TreeCand { float score; int depth, rank, parent; };

__global__ __launch_bounds__(TREE_THREADS) void tree_build_kernel(const float *topk_val, const int *topk_idx,
                                                                  const int *anchor, int batch, int B, int K, int N,
                                                                  int *tree_tok, int *tree_parent) {
  __shared__ TreeCand heap_sh[2 * TREE_MAX_NODES + 2][TREE_THREADS];
  __shared__ float nscore_sh[TREE_MAX_NODES][TREE_THREADS];
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= batch) return;
  using Cand = TreeCand;
  auto heap_at = [&](int i) -> Cand & { return heap_sh[i][threadIdx.x]; };
  auto nscore = [&](int i) -> float & { return nscore_sh[i][threadIdx.x]; };
  int hn = 0;
  auto better = [](const Cand &a, const Cand &b) {
    if (a.score != b.score) return a.score > b.score;
    if (a.depth != b.depth) return a.depth < b.depth;
    return a.rank < b.rank;
  };
  auto push = [&](Cand c) {
    int i = hn++;
    while (i > 0) {
      const int pi = (i - 1) / 2;
      if (!better(c, heap_at(pi))) break;
      heap_at(i) = heap_at(pi);
      i = pi;
    }
    heap_at(i) = c;
  };
  auto pop = [&]() {
    const Cand top = heap_at(0);
    const Cand last = heap_at(--hn);
    int i = 0;
    while (true) {
      int c = 2 * i + 1;
      if (c >= hn) break;
      if (c + 1 < hn && better(heap_at(c + 1), heap_at(c))) ++c;
      if (!better(heap_at(c), last)) break;
      heap_at(i) = heap_at(c);
      i = c;
    }
    if (hn > 0) heap_at(i) = last;
    return top;
  };
  const float *val = topk_val + size_t(s) * B * K;
  const int *idx = topk_idx + size_t(s) * B * K;
  int *tok = tree_tok + size_t(s) * (N + 1);
  int *par = tree_parent + size_t(s) * (N + 1);
  tok[0] = anchor[s];
  par[0] = -1;
  nscore(0) = 0.f;
  push(Cand{val[0], 1, 0, 0});
  int nodes = 1;
  while (hn > 0 && nodes < N + 1) {
    const Cand c = pop();
    const int node = nodes++;
    tok[node] = idx[(c.depth - 1) * K + c.rank];
    par[node] = c.parent;
    nscore(node) = c.score;
    if (c.rank + 1 < K) push(Cand{nscore(c.parent) + val[(c.depth - 1) * K + c.rank + 1], c.depth, c.rank + 1, c.parent});
    if (c.depth < B) push(Cand{c.score + val[c.depth * K], c.depth + 1, 0, node});
  }
  for (; nodes < N + 1; ++nodes) {   // fewer continuations than N: a chain of repeats is never produced
    tok[nodes] = tok[0];
    par[nodes] = 0;
  }
}

__global__ __launch_bounds__(TREE_THREADS) void tree_prep_kernel(const int *parent, int batch, int n, int *depth,
                                                                 unsigned *mask, unsigned *status) {
  __shared__ int dep_sh[TREE_MAX_NODES][TREE_THREADS];
  __shared__ unsigned msk_sh[TREE_MAX_NODES][TREE_THREADS];
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= batch) return;
  const int *par = parent + size_t(s) * n;
  auto dep = [&](int i) -> int & { return dep_sh[i][threadIdx.x]; };
  auto msk = [&](int i) -> unsigned & { return msk_sh[i][threadIdx.x]; };
  bool bad = false;
  for (int i = 0; i < n; ++i) {
    int pi = par[i];
    if (i == 0) {
      bad = bad || pi != -1;
      dep(0) = 0;
      msk(0) = 1u;
    } else {
      if (pi < 0 || pi >= i) {
        bad = true;
        pi = i - 1;
      }
      dep(i) = dep(pi) + 1;
      msk(i) = msk(pi) | (1u << i);
    }
    depth[s * n + i] = dep(i);
    mask[s * n + i] = msk(i);
  }
  if (bad) atomicOr(status, DFLASH_STATUS_TREE);
}

__global__ void tree_walk_kernel(const int *tree_tok, const int *parent, const int *target_argmax, int batch, int n,
                                 int *accept_len, int *bonus, int *path) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= batch) return;
  const int *tok = tree_tok + size_t(s) * n;
  const int *par = parent + size_t(s) * n;
  const int *g = target_argmax + size_t(s) * n;
  int *pth = path + size_t(s) * n;
  int node = 0, L = 0;
  pth[0] = 0;
  while (true) {
    int next = -1;
    for (int c = node + 1; c < n; ++c)
      if (par[c] == node && tok[c] == g[node]) {
        next = c;
        break;
      }
    if (next < 0) break;
    node = next;
    pth[++L] = node;
  }
  for (int k = L + 1; k < n; ++k) pth[k] = -1;
  accept_len[s] = L;
  bonus[s] = g[node];
}

// One workgroup per (layer, sequence, KV head): the path rows are read into
// LDS first, then written to their new slots (a source slot can be another
// row's destination).
template <typename T>
__global__ __launch_bounds__(256) void commit_path_kernel(char *kcache, char *vcache, const int *ctx_len, const int *path,
                                                          const int *accept_len, int n, int max_batch, int n_kv,
                                                          int capacity, int head_dim) {
  __shared__ float kv[2][TREE_MAX_NODES][128];
  const int g = blockIdx.x, s = blockIdx.y, l = blockIdx.z;
  const int C = ctx_len[s], L = min(max(accept_len[s], 0), n - 1);
  const size_t region = size_t(capacity) * head_dim * Ty<T>::SIZE;
  char *kreg = kcache + ((size_t(l) * max_batch + s) * n_kv + g) * region;
  char *vreg = vcache + ((size_t(l) * max_batch + s) * n_kv + g) * region;
  for (int e = threadIdx.x; e < (L + 1) * head_dim; e += blockDim.x) {
    const int k = e / head_dim, dd = e % head_dim;
    const int src = min(C + max(path[s * n + k], 0), capacity - 1);
    kv[0][k][dd] = to_f32<T>(*reinterpret_cast<const T *>(kreg + kcache_offset<T>(src, dd, head_dim)));
    kv[1][k][dd] = to_f32<T>(*reinterpret_cast<const T *>(vreg + vcache_offset<T>(src, dd, head_dim)));
  }
  __syncthreads();
  for (int e = threadIdx.x; e < (L + 1) * head_dim; e += blockDim.x) {
    const int k = e / head_dim, dd = e % head_dim;
    const int dst = C + k;
    if (dst < capacity) {
      store_elem<T>(kreg + kcache_offset<T>(dst, dd, head_dim), kv[0][k][dd]);
      store_elem<T>(vreg + vcache_offset<T>(dst, dd, head_dim), kv[1][k][dd]);
    }
  }
}

__global__ void commit_len_kernel(int *ctx_len, const int *accept_len, int batch, int n, int capacity) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= batch) return;
  ctx_len[s] = min(ctx_len[s] + min(max(accept_len[s], 0), n - 1) + 1, capacity);
}

hipError_t launch_row_topk(const float *logits, int ld, int vocab, int rows, int K, const float *lse,
                           unsigned long long *chunk_keys, float *topk_val, int *topk_idx, hipStream_t s) {
  if (K < 1 || K > TREE_MAX_K || TOPK_CHUNKS * K > TOPK_THREADS * TREE_MAX_K) return hipErrorInvalidValue;
  hipLaunchKernelGGL(row_topk_part_kernel, dim3(TOPK_CHUNKS, rows), dim3(TOPK_THREADS), 0, s, logits, ld, vocab, K,
                     chunk_keys);
  hipLaunchKernelGGL(row_topk_merge_kernel, dim3(rows), dim3(TOPK_THREADS), 0, s, logits, ld, vocab, K, chunk_keys,
                     lse, topk_val, topk_idx);
  return hipGetLastError();
}

hipError_t launch_tree_build(const float *topk_val, const int *topk_idx, const int *anchor, int batch, int B,
                             int K, int N, int *tree_tok, int *tree_parent, hipStream_t s) {
  if (K < 1 || K > TREE_MAX_K || N < 1 || N + 1 > TREE_MAX_NODES) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tree_build_kernel, dim3((batch + TREE_THREADS - 1) / TREE_THREADS), dim3(TREE_THREADS), 0, s,
                     topk_val, topk_idx, anchor, batch,
                     B, K, N, tree_tok, tree_parent);
  return hipGetLastError();
}

hipError_t launch_tree_prep(const int *parent, int batch, int n, int *depth, unsigned *mask, unsigned *status,
                            hipStream_t s) {
  if (n < 1 || n > TREE_MAX_NODES) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tree_prep_kernel, dim3((batch + TREE_THREADS - 1) / TREE_THREADS), dim3(TREE_THREADS), 0, s,
                     parent, batch, n, depth, mask, status);
  return hipGetLastError();
}

hipError_t launch_tree_walk(const int *tree_tok, const int *parent, const int *target_argmax, int batch, int n,
                            int *accept_len, int *bonus, int *path, hipStream_t s) {
  hipLaunchKernelGGL(tree_walk_kernel, dim3((batch + 63) / 64), dim3(64), 0, s, tree_tok, parent, target_argmax,
                     batch, n, accept_len, bonus, path);
  return hipGetLastError();
}

hipError_t launch_commit_path(int dtype, char *kcache, char *vcache, int *ctx_len, const int *path,
                              const int *accept_len, int batch, int n, int n_layers, int max_batch, int n_kv,
                              int capacity, int head_dim, hipStream_t s) {
  if (n < 1 || n > TREE_MAX_NODES || head_dim > 128) return hipErrorInvalidValue;
  const dim3 grid(n_kv, batch, n_layers);
  if (dtype == DFLASH_BF16)
    hipLaunchKernelGGL(commit_path_kernel<bf16_t>, grid, dim3(256), 0, s, kcache, vcache, ctx_len, path, accept_len,
                       n, max_batch, n_kv, capacity, head_dim);
  else
    hipLaunchKernelGGL(commit_path_kernel<float>, grid, dim3(256), 0, s, kcache, vcache, ctx_len, path, accept_len,
                       n, max_batch, n_kv, capacity, head_dim);
  hipLaunchKernelGGL(commit_len_kernel, dim3((batch + 63) / 64), dim3(64), 0, s, ctx_len, accept_len, batch, n,
                     capacity);
  return hipGetLastError();
}

}  // namespace dflash
