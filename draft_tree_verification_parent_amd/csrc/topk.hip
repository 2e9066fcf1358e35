// Vocabulary-wide top-k per row (ties to the lower id); argmax = column 0.
//
// The successor table keeps each token's k most likely successors and greedy
// acceptance compares draft tokens with the target's most likely token
// (Graft page, arXiv:2605.20104 write-up, section 2, second and third
// steps); both read one per-row top-k of the fp32 logits.
//
// Two passes, both bound by the read of the logits:
//  1. grid (slices, rows): each thread keeps a sorted top-K list in
//     registers over its strided part of a slice (coalesced float4 reads),
//     each wavefront merges its 64 lists with k rounds of a (value, id)
//     butterfly max, and wave 0 merges the four wave results; k candidates
//     per (row, slice) go to the workspace.
//  2. one wavefront per row merges the slices' candidates the same way.
// The (value desc, id asc) order is total on non-NaN values, so the result
// does not depend on how the vocabulary is split.
#include <climits>

#include "common.h"
#include "kernels.h"

namespace {

constexpr int kThreads = 256;
constexpr int kSliceQuantum = 1024;  // 256 threads x float4

template <int K>
struct TopList {
  float v[K];
  int id[K];
  __device__ void init() {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      v[j] = -INFINITY;
      id[j] = INT_MAX;
    }
  }
  __device__ void insert(float x, int i) {
    if (!graft::better(x, i, v[K - 1], id[K - 1])) return;
    v[K - 1] = x;
    id[K - 1] = i;
#pragma unroll
    for (int j = K - 1; j > 0; --j) {
      const bool sw = graft::better(v[j], id[j], v[j - 1], id[j - 1]);
      const float tv = v[j - 1];
      const int ti = id[j - 1];
      v[j - 1] = sw ? v[j] : tv;
      id[j - 1] = sw ? id[j] : ti;
      v[j] = sw ? tv : v[j];
      id[j] = sw ? ti : id[j];
    }
  }
  __device__ void pop_front() {
#pragma unroll
    for (int j = 0; j < K - 1; ++j) {
      v[j] = v[j + 1];
      id[j] = id[j + 1];
    }
    v[K - 1] = -INFINITY;
    id[K - 1] = INT_MAX;
  }
};

// Best (value, id) over the 64 lanes; every lane gets the result.
__device__ inline void wave_best(float &bv, int &bi) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    if (graft::better(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
}

// k rounds of extraction from per-lane sorted lists; lane j < k returns the
// j-th best in (out_v, out_i).
template <int K>
__device__ void wave_extract(TopList<K> &L, int k, float &out_v, int &out_i) {
  const int lane = threadIdx.x & 63;
  out_v = -INFINITY;
  out_i = INT_MAX;
  for (int j = 0; j < k; ++j) {
    float bv = L.v[0];
    int bi = L.id[0];
    wave_best(bv, bi);
    if (L.id[0] == bi && L.v[0] == bv) L.pop_front();
    if (lane == j) {
      out_v = bv;
      out_i = bi;
    }
  }
}

template <int K>
__global__ __launch_bounds__(kThreads) void topk_slice_kernel(const float *__restrict__ logits, int V, int k,
                                                              int slice_len, float *__restrict__ part_v,
                                                              int *__restrict__ part_i,
                                                              int32_t *__restrict__ out_id,
                                                              float *__restrict__ out_val) {
  __shared__ float s_v[4][GRAFT_MAX_K];
  __shared__ int s_i[4][GRAFT_MAX_K];
  const int s = blockIdx.x;
  const int S = gridDim.x;
  const int m = blockIdx.y;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const float *row = logits + static_cast<size_t>(m) * V;
  const int lo = s * slice_len;
  const int hi = lo + slice_len < V ? lo + slice_len : V;

  TopList<K> L;
  L.init();
  if ((V & 3) == 0) {
    for (int c = lo + tid * 4; c < hi; c += kThreads * 4) {
      const float4 x = *reinterpret_cast<const float4 *>(row + c);
      L.insert(x.x, c);
      L.insert(x.y, c + 1);
      L.insert(x.z, c + 2);
      L.insert(x.w, c + 3);
    }
  } else {
    for (int c = lo + tid; c < hi; c += kThreads) L.insert(row[c], c);
  }

  float rv;
  int ri;
  wave_extract<K>(L, k, rv, ri);
  if (lane < k) {
    s_v[wave][lane] = rv;
    s_i[wave][lane] = ri;
  }
  __syncthreads();
  if (wave == 0) {
    TopList<K> M;
    M.init();
    if (lane < 4 * k) M.insert(s_v[lane / k][lane % k], s_i[lane / k][lane % k]);
    wave_extract<K>(M, k, rv, ri);
    if (lane < k) {
      if (S == 1) {
        out_id[static_cast<size_t>(m) * k + lane] = ri == INT_MAX ? 0 : ri;
        if (out_val) out_val[static_cast<size_t>(m) * k + lane] = rv;
      } else {
        const size_t o = (static_cast<size_t>(m) * S + s) * k + lane;
        part_v[o] = rv;
        part_i[o] = ri;
      }
    }
  }
}

template <int K>
__global__ __launch_bounds__(64) void topk_merge_kernel(int S, int k, const float *__restrict__ part_v,
                                                        const int *__restrict__ part_i,
                                                        int32_t *__restrict__ out_id,
                                                        float *__restrict__ out_val) {
  const int m = blockIdx.x;
  const int lane = threadIdx.x;
  const size_t base = static_cast<size_t>(m) * S * k;
  TopList<K> L;
  L.init();
  for (int c = lane; c < S * k; c += 64) L.insert(part_v[base + c], part_i[base + c]);
  float rv;
  int ri;
  wave_extract<K>(L, k, rv, ri);
  if (lane < k) {
    out_id[static_cast<size_t>(m) * k + lane] = ri == INT_MAX ? 0 : ri;
    if (out_val) out_val[static_cast<size_t>(m) * k + lane] = rv;
  }
}

}  // namespace

namespace graft {

TopkPlan topk_plan(int M, int V, int k) {
  TopkPlan p;
  const int max_slices = (V + kSliceQuantum - 1) / kSliceQuantum;
  int want = M > 0 ? (1024 + M - 1) / M : 1;
  if (want < 1) want = 1;
  if (want > max_slices) want = max_slices;
  int per = (V + want - 1) / want;
  per = (per + kSliceQuantum - 1) / kSliceQuantum * kSliceQuantum;
  p.slice_len = per;
  p.slices = (V + per - 1) / per;
  p.ws_bytes = p.slices > 1 ? static_cast<size_t>(M) * p.slices * k * (sizeof(float) + sizeof(int)) : 0;
  return p;
}

int launch_topk(int M, int V, int k, const float *logits, int32_t *topk_id, float *topk_val, void *ws,
                hipStream_t stream) {
  const TopkPlan p = topk_plan(M, V, k);
  float *part_v = static_cast<float *>(ws);
  int *part_i = reinterpret_cast<int *>(part_v + static_cast<size_t>(M) * p.slices * k);
  dim3 grid(p.slices, M);
  if (k <= 8) {
    hipLaunchKernelGGL(topk_slice_kernel<8>, grid, dim3(kThreads), 0, stream, logits, V, k, p.slice_len,
                       part_v, part_i, topk_id, topk_val);
    if (p.slices > 1)
      hipLaunchKernelGGL(topk_merge_kernel<8>, dim3(M), dim3(64), 0, stream, p.slices, k, part_v, part_i,
                         topk_id, topk_val);
  } else {
    hipLaunchKernelGGL(topk_slice_kernel<16>, grid, dim3(kThreads), 0, stream, logits, V, k, p.slice_len,
                       part_v, part_i, topk_id, topk_val);
    if (p.slices > 1)
      hipLaunchKernelGGL(topk_merge_kernel<16>, dim3(M), dim3(64), 0, stream, p.slices, k, part_v, part_i,
                         topk_id, topk_val);
  }
  return check_launch("topk");
}

}  // namespace graft
