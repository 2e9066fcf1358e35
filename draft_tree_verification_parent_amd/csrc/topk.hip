// Vocabulary-wide top-k per row (ties to the lower id); argmax = column 0.
//
// The successor table keeps each token's k most likely successors and greedy
// acceptance compares draft tokens with the target's most likely token
// (Graft page, arXiv:2605.20104 write-up, section 2, second and third
// steps); both read one per-row top-k of the fp32 logits.
//
// Two passes, both bound by the read of the logits:
//  1. grid (slices, rows): each thread keeps a sorted top-K list in
//     registers over its strided part of a slice (coalesced float4 reads;
//     a batch runs inserts only when its largest entry passes a wave-wide
//     bound, so that after the first batches almost none does),
//     each wavefront merges its 64 lists with k rounds of a (value, id)
//     butterfly max, and wave 0 merges the four wave results; k candidates
//     per (row, slice) go to the workspace.
//  2. one workgroup per row merges the slices' candidates the same way
//     (not needed with one slice per row, the case past 256 rows).
// The (value desc, id asc) order is total on non-NaN values, so the result
// does not depend on how the vocabulary is split.
#include <climits>

#include "common.h"
#include "kernels.h"
#include "topk_list.h"

namespace {

constexpr int kThreads = 256;
constexpr int kSliceQuantum = 4;  // slices start on 16-byte boundaries

using graft::TopKeys;

typedef float f32x4 __attribute__((ext_vector_type(4)));
// Four logits (16 bytes) read once: a non-temporal load (the logits are not read again,
// and the stream runs at 0.77 of HBM peak this way against 0.70 cached).
__device__ inline float4 load_stream4(const float *p) {
  const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
  return make_float4(t[0], t[1], t[2], t[3]);
}

template <int K>
__global__ __launch_bounds__(kThreads) void topk_slice_kernel(const float *__restrict__ logits, int V, int k,
                                                              int slice_len, uint64_t *__restrict__ part,
                                                              int32_t *__restrict__ out_id,
                                                              float *__restrict__ out_val) {
  __shared__ uint64_t s_k[4][GRAFT_MAX_K];
  const int s = blockIdx.x;
  const int S = gridDim.x;
  const int m = blockIdx.y;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const float *row = logits + static_cast<size_t>(m) * V;
  const int lo = s * slice_len;
  const int hi = lo + slice_len < V ? lo + slice_len : V;

  // one sorted list per lane, fp64 keys: an insert is K v_max_f64 /
  // v_min_f64 pairs (ids below 2^30, which the host checks)
  graft::F64Keys<K> L;
  L.init();
  // Each wave's bound, published for the others: an entry below any wave's
  // bound is below K entries of the row, so every wave screens with the
  // largest published one (a stale value is still a valid bound).
  __shared__ uint32_t s_bound[4];
  if (tid < 4) s_bound[tid] = 0;
  __syncthreads();
  // An entry below a value that K distinct entries of the wave reach cannot
  // be in the top k <= K.  `bound` (a value order) is the K-th largest of the
  // 64 lanes' list heads after each batch, and of the lanes' maxima before
  // the first: it follows the wave's own K-th largest entry, so after the
  // first batches almost every entry fails this one compare and a batch's
  // 16 slots rarely run an insert.  (A uniform trip count keeps all 64 lanes
  // in the cross-lane max.)
  uint32_t bound = 0;
  // 16-byte loads per thread per batch, issued together (8 for the longer
  // lists measured slower once their bound update was a sort)
  constexpr int U = 4;
  if ((V & 3) == 0) {
    // Whole batches need no bounds checks.  The screen is a float compare
    // against the bound's value, !(x < bf): for numbers it is order(x) >=
    // bound; while the bound is 0 (no lane full yet) bf is a NaN and every
    // entry passes; a NaN entry passes too, and the list's own key compare
    // then keeps it out unless the list has room (NaN ranks last).  A batch
    // runs its inserts, and the bound is raised, only when the wave's
    // largest entry passes, which after the first batches is rare.
    constexpr int B = kThreads * 4 * U;
    int base = lo;
    float bf = __uint_as_float(0xFFFFFFFFu);  // the value of order 0: a NaN
    // The next batch's loads are issued before this batch is screened, so
    // each workgroup always has a batch in flight.
    float4 x[U], xn[U];
    if (base + B <= hi) {
#pragma unroll
      for (int u = 0; u < U; ++u) xn[u] = load_stream4(row + base + (u * kThreads + tid) * 4);
    }
    for (; base + B <= hi; base += B) {
#pragma unroll
      for (int u = 0; u < U; ++u) x[u] = xn[u];
      if (base + 2 * B <= hi) {  // uniform
#pragma unroll
        for (int u = 0; u < U; ++u)
          xn[u] = load_stream4(row + base + B + (u * kThreads + tid) * 4);
      }
      if (base == lo) {
        // first batch (uniform): the K-th largest of the 64 lane maxima, so
        // the first inserts are already filtered
        uint32_t lm = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float xs[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t o = graft::float_order(xs[e]);
            lm = o > lm ? o : lm;
          }
        }
        bound = graft::wave_kth_u32<K>(lm);
        bf = graft::key_value(static_cast<uint64_t>(bound) << 32);
        if (lane == 0) __hip_atomic_store(&s_bound[wave], bound, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      {
        // relaxed atomic loads: other waves store these meanwhile
        uint32_t ob = 0;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2)
          ob = max(ob, __hip_atomic_load(&s_bound[w2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
        if (ob > bound) {
          bound = ob;
          bf = graft::key_value(static_cast<uint64_t>(bound) << 32);
        }
      }
      float mx = fmaxf(fmaxf(x[0].x, x[0].y), fmaxf(x[0].z, x[0].w));
#pragma unroll
      for (int u = 1; u < U; ++u) mx = fmaxf(mx, fmaxf(fmaxf(x[u].x, x[u].y), fmaxf(x[u].z, x[u].w)));
      // (fmaxf drops NaNs unless all are: a batch whose numbers all fail
      // skips its NaNs, which rank below them)
      if (__builtin_amdgcn_ballot_w64(!(mx < bf)) == 0) continue;  // uniform
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = base + (u * kThreads + tid) * 4;
        const float xs[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (!(xs[e] < bf)) L.insert(graft::F64Keys<K>::make(xs[e], c + e));
      }
      // each lane's list head is its largest entry: K lanes hold an entry
      // at least the K-th largest head
      const uint32_t lb = graft::wave_kth_u32<K>(L.head_order());
      if (lb > bound) {
        bound = lb;
        bf = graft::key_value(static_cast<uint64_t>(bound) << 32);
        if (lane == 0) __hip_atomic_store(&s_bound[wave], bound, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
    // the partial batch at the end of the slice, entry by entry
    for (; base < hi; base += kThreads * 4) {
      const int c = base + tid * 4;
      if (c < hi) {
        const float4 v = *reinterpret_cast<const float4 *>(row + c);
        const float xs[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (c + e < hi && graft::float_order(xs[e]) >= bound) L.insert(graft::F64Keys<K>::make(xs[e], c + e));
      }
    }
  } else {
    for (int base = lo; base < hi; base += kThreads * U) {
      float x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = base + u * kThreads + tid;
        x[u] = c < hi ? row[c] : 0.f;
      }
      if (base == lo) {
        uint32_t lm = 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint32_t o = base + u * kThreads + tid < hi ? graft::float_order(x[u]) : 0u;
          lm = o > lm ? o : lm;
        }
        bound = graft::wave_kth_u32<K>(lm);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = base + u * kThreads + tid;
        if (c < hi && graft::float_order(x[u]) >= bound) L.insert(graft::F64Keys<K>::make(x[u], c));
      }
      // each lane's list head is its largest entry: K lanes hold an entry
      // at least the K-th largest head
      const uint32_t lb = graft::wave_kth_u32<K>(L.head_order());
      bound = lb > bound ? lb : bound;
    }
  }

  TopKeys<K> LK;  // the lane's list as rank keys
#pragma unroll
  for (int j = 0; j < K; ++j) LK.k[j] = L.rank_key(j);
  uint64_t r = graft::wave_extract<K>(LK, k);
  if (lane < k) s_k[wave][lane] = r;
  __syncthreads();
  if (wave == 0) {
    TopKeys<K> M2;
    M2.init();
    if (lane < 4 * k) M2.insert(s_k[lane / k][lane % k]);
    r = graft::wave_extract<K>(M2, k);
    if (lane < k) {
      if (S == 1) {
        out_id[static_cast<size_t>(m) * k + lane] = r ? graft::key_id(r) : 0;
        if (out_val) out_val[static_cast<size_t>(m) * k + lane] = r ? graft::key_value(r) : -INFINITY;
      } else {
        part[(static_cast<size_t>(m) * S + s) * k + lane] = r;
      }
    }
  }
}

// One 256-thread workgroup per row.  With at most 256 candidate lists a
// thread takes one list as its own sorted list (the producers write each
// list largest first); otherwise each thread ranks ~1/256 of the row's
// candidates (loads batched 8 at a time so their latencies overlap).  Each
// wavefront extracts its k best, and wave 0 merges the four wave results.
template <int K>
__global__ __launch_bounds__(kThreads) void topk_merge_kernel(int S, int k, const uint64_t *__restrict__ part,
                                                              int32_t *__restrict__ out_id,
                                                              float *__restrict__ out_val) {
  __shared__ uint64_t s_k[4][GRAFT_MAX_K];
  const int m = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const uint64_t *row = part + static_cast<size_t>(m) * S * k;
  const int n = S * k;
  TopKeys<K> L;
  L.init();
  if (S <= kThreads) {
    // every producer writes its k keys sorted (largest first): thread t
    // takes list t as its own, no inserts needed
    if (tid < S) {
      const uint64_t *lst = row + static_cast<size_t>(tid) * k;
#pragma unroll
      for (int j = 0; j < K; ++j) L.k[j] = j < k ? lst[j] : 0;
    }
  } else {
    constexpr int BATCH = 8;
    for (int c0 = 0; c0 < n; c0 += kThreads * BATCH) {
      uint64_t x[BATCH];
#pragma unroll
      for (int j = 0; j < BATCH; ++j) {
        const int c = c0 + j * kThreads + tid;
        x[j] = c < n ? row[c] : 0;
      }
#pragma unroll
      for (int j = 0; j < BATCH; ++j) L.insert(x[j]);
    }
  }
  uint64_t r = graft::wave_extract<K>(L, k);
  if (lane < k) s_k[wave][lane] = r;
  __syncthreads();
  if (wave == 0) {
    TopKeys<K> M2;
    M2.init();
    if (lane < 4 * k) M2.insert(s_k[lane / k][lane % k]);
    r = graft::wave_extract<K>(M2, k);
    if (lane < k) {
      out_id[static_cast<size_t>(m) * k + lane] = r ? graft::key_id(r) : 0;
      if (out_val) out_val[static_cast<size_t>(m) * k + lane] = r ? graft::key_value(r) : -INFINITY;
    }
  }
}

// At most 64 candidate lists per row (a sliced top-k of a vocabulary up to
// 64 x 4096 entries, and the 256 x 256 lm-head kernel from four m tiles on,
// which writes one list per tile stream): one wavefront per row, four rows
// per workgroup; lane t takes list t as its own and the wavefront extracts
// the k best.  The same keys as topk_merge_kernel, whose other three
// wavefronts would hold only empty lists.
template <int K>
__global__ __launch_bounds__(kThreads) void topk_merge_wave_kernel(int M, int S, int k,
                                                                   const uint64_t *__restrict__ part,
                                                                   int32_t *__restrict__ out_id,
                                                                   float *__restrict__ out_val) {
  const int m = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (m >= M) return;  // the whole wavefront
  TopKeys<K> L;
  L.init();
  if (lane < S) {
    const uint64_t *lst = part + (static_cast<size_t>(m) * S + lane) * k;
#pragma unroll
    for (int j = 0; j < K; ++j) L.k[j] = j < k ? lst[j] : 0;
  }
  const uint64_t r = graft::wave_extract<K>(L, k);
  if (lane < k) {
    out_id[static_cast<size_t>(m) * k + lane] = r ? graft::key_id(r) : 0;
    if (out_val) out_val[static_cast<size_t>(m) * k + lane] = r ? graft::key_value(r) : -INFINITY;
  }
}

// One draw per row at temperature T by the Gumbel-max identity on
// materialised logits: argmax_t fl(fl(l_t * inv_temp) + g_t), ties to the
// lower id, NaN below every number.  One 256-thread workgroup per row.
__global__ __launch_bounds__(kThreads) void sample_rows_kernel(int V, float inv_temp, const float *__restrict__ logits,
                                                               const float *__restrict__ gumbel,
                                                               int32_t *__restrict__ sample_id) {
  __shared__ uint64_t s_best[kThreads / 64];
  const int m = blockIdx.x;
  const int tid = threadIdx.x;
  const float *lr = logits + static_cast<size_t>(m) * V;
  const float *gr = gumbel + static_cast<size_t>(m) * V;
  uint64_t best = 0;
  for (int t0 = 0; t0 < V; t0 += kThreads * 4) {
    float l[4], g[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = t0 + u * kThreads + tid;
      l[u] = t < V ? lr[t] : 0.f;
      g[u] = t < V ? gr[t] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      // two roundings, as defined: no fused multiply-add
#pragma clang fp contract(off)
      const int t = t0 + u * kThreads + tid;
      if (t < V) {
        const float scaled = l[u] * inv_temp;
        float sc = scaled + g[u];
        sc = sc != sc ? -INFINITY : sc;
        const uint64_t key = graft::rank_key(sc, t);
        best = key > best ? key : best;
      }
    }
  }
  best = graft::group_max<64>(best);
  if ((tid & 63) == 0) s_best[tid >> 6] = best;
  __syncthreads();
  if (tid == 0) {
    uint64_t b = s_best[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) b = s_best[w] > b ? s_best[w] : b;
    sample_id[m] = graft::key_id(b);
  }
}

}  // namespace

namespace graft {

TopkPlan topk_plan(int M, int V, int k) {
  TopkPlan p;
  // at least one workgroup per CU, slices of equal length (at least 4096
  // entries: a slice's first batch sets its bound).  Past 256 rows one
  // workgroup per row: more slices measured slower (960 x 151936 fp32
  // logits, cold, with an earlier version of the slice kernel: 110 us with
  // one slice per row, 119 with two, 121 with four; k = 16: 141, 174, 222),
  // each adding its own bound set-up, list extraction and merge.
  const int max_slices = (V + 4095) / 4096;
  int want = M > 0 ? (256 + M - 1) / M : 1;
  if (want > max_slices) want = max_slices;
  if (want < 1) want = 1;
  int per = (V + want - 1) / want;
  per = (per + kSliceQuantum - 1) / kSliceQuantum * kSliceQuantum;
  p.slice_len = per;
  p.slices = (V + per - 1) / per;
  p.ws_bytes = p.slices > 1 ? static_cast<size_t>(M) * p.slices * k * sizeof(uint64_t) : 0;
  return p;
}

int launch_topk(int M, int V, int k, const float *logits, int32_t *topk_id, float *topk_val, void *ws,
                hipStream_t stream) {
  const TopkPlan p = topk_plan(M, V, k);
  uint64_t *part = static_cast<uint64_t *>(ws);
  dim3 grid(p.slices, M);
  if (k <= 8)
    hipLaunchKernelGGL(topk_slice_kernel<8>, grid, dim3(kThreads), 0, stream, logits, V, k, p.slice_len, part,
                       topk_id, topk_val);
  else
    hipLaunchKernelGGL(topk_slice_kernel<16>, grid, dim3(kThreads), 0, stream, logits, V, k, p.slice_len, part,
                       topk_id, topk_val);
  if (p.slices > 1) return launch_topk_merge(M, p.slices, k, part, topk_id, topk_val, stream);
  return check_launch("topk");
}

int launch_topk_merge(int M, int slices, int k, const uint64_t *part, int32_t *topk_id, float *topk_val,
                      hipStream_t stream) {
  if (slices <= 64) {
    const dim3 grid((M + kThreads / 64 - 1) / (kThreads / 64));
    if (k <= 8)
      hipLaunchKernelGGL(topk_merge_wave_kernel<8>, grid, dim3(kThreads), 0, stream, M, slices, k, part, topk_id,
                         topk_val);
    else
      hipLaunchKernelGGL(topk_merge_wave_kernel<16>, grid, dim3(kThreads), 0, stream, M, slices, k, part, topk_id,
                         topk_val);
    return check_launch("topk merge");
  }
  if (k <= 8)
    hipLaunchKernelGGL(topk_merge_kernel<8>, dim3(M), dim3(kThreads), 0, stream, slices, k, part, topk_id, topk_val);
  else
    hipLaunchKernelGGL(topk_merge_kernel<16>, dim3(M), dim3(kThreads), 0, stream, slices, k, part, topk_id,
                       topk_val);
  return check_launch("topk merge");
}

}  // namespace graft

extern "C" int graft_sample_rows(int M, int V, float temperature, const float *logits, const float *gumbel,
                                 int32_t *sample_id, graft_stream stream) {
  using graft::fail;
  if (M < 0 || V <= 0 || M > 0x7FFFFFFF) return fail(GRAFT_EINVAL, "sample_rows: M=%d V=%d", M, V);
  if (!(temperature > 0.f) || !(temperature < INFINITY))
    return fail(GRAFT_EINVAL, "sample_rows: temperature must be positive and finite");
  if (M == 0) return GRAFT_OK;
  if (!logits || !gumbel || !sample_id) return fail(GRAFT_EINVAL, "sample_rows: NULL array");
  graft::clear_error();
  hipLaunchKernelGGL(sample_rows_kernel, dim3(M), dim3(kThreads), 0, graft::as_stream(stream), V, 1.0f / temperature,
                     logits, gumbel, sample_id);
  return graft::check_launch("sample_rows");
}
