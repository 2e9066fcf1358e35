// lm-head GEMM: logits[m, v] = sum_h hidden[m, h] * W[v, h], bf16 in, fp32 out,
// optionally fused with the per-row top-k so the logits never reach HBM.
//
// The verification pass ends in each tree position's next-token
// distribution, which the table update and the acceptance test read (Graft
// page, arXiv:2605.20104 write-up, section 2, third step).
//
// With M = tree nodes (tens) and V x H = 0.5-0.8 G weights, this is a
// weight-streaming product bound by HBM (about 60 flop per weight byte).
// V_MFMA_F32_16X16X32_BF16 computes 16 vocabulary rows x 16 hidden rows.
//
// Two weight layouts:
//  * packed (graft_lmhead_pack, done once when the weights are loaded): W
//    is cut into images of 128 vocabulary rows x 64 hidden columns (16 KB,
//    row-major inside), stored tile by tile, column chunk by column chunk,
//    so a workgroup's whole weight stream is one contiguous, linearly read
//    region whatever its stage width.  A persistent grid (one workgroup per
//    CU) copies images HBM -> LDS with global_load_lds_dwordx4 (LDS DMA: no
//    registers, in a ring that runs across tile boundaries), stages the
//    hidden chunk the same way, and reads both MFMA operands from LDS.  The
//    DMA lands 16 bytes per lane at consecutive LDS addresses, and the
//    per-lane source offsets pick which piece lands where: LDS rows are
//    XOR-swizzled so 16 lanes reading one MFMA fragment column hit 16
//    different bank groups.  Linear reads reach about 7.2 TB/s on MI355X
//    where row-major tiles (256-byte runs per row) stall near 5.6 TB/s, and
//    128-byte runs at a 256-byte stride near 3.2 TB/s.
//  * row-major W [V, H]: W read straight from HBM into MFMA operand
//    registers (ping-pong buffers), the hidden chunk double-buffered in LDS.
// Fused top-k: each logit tile goes through LDS and 4 threads per row rank
// 32 entries each into sorted register lists of 64-bit (value, id) keys; k
// keys per (row, list owner) are written and a second kernel merges them
// (the (value desc, id asc) order is total, so the result does not depend
// on the split).  In the packed path the lists persist across a
// workgroup's tiles, so the merge reads one list per (row, workgroup).
#include <climits>
#include <mutex>
#include <type_traits>
#include <utility>

#include "common.h"
#include "kernels.h"
#include "topk_list.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBV = kWaves * 32;

__device__ inline bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

// f(integral_constant<int, i>) for i = 0 .. N - 1, unrolled at compile time
template <typename F, int... I>
__device__ inline void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ inline void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}
__device__ inline u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

template <int KC, bool FUSED, int K>
__global__ __launch_bounds__(kThreads, 4) void lmhead_kernel(int M, int H, int V, int k,
                                                           const graft_bf16 *__restrict__ hidden,
                                                           const graft_bf16 *__restrict__ w,
                                                           float *__restrict__ logits,
                                                           uint64_t *__restrict__ part_out, int tiles_m,
                                                           int tiles_v) {
  constexpr int WAVES = kWaves;
  constexpr int BV = kBV;
  constexpr int STR = KC + 8;             // bf16 per staged hidden row (16 B pad)
  constexpr int KS = KC / 32;             // MFMA k-steps per chunk
  constexpr int PPT = BM * KC / 8 / kThreads;  // hidden 16-byte pieces staged per thread
  constexpr int TSTR = BV + 4;            // floats per row of the fused top-k logit tile
  constexpr int STAGE_BYTES = 2 * BM * STR * 2;
  constexpr int TILE_BYTES = FUSED ? BM * TSTR * 4 : 0;
  __shared__ __attribute__((aligned(16))) unsigned char smem[STAGE_BYTES > TILE_BYTES ? STAGE_BYTES : TILE_BYTES];
  graft_bf16(*s_h)[BM * STR] = reinterpret_cast<graft_bf16(*)[BM * STR]>(smem);

  const int total = tiles_m * tiles_v;
  const int per_xcd = (total + 7) / 8;
  const int logical = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (logical >= total) return;
  const int tm = logical % tiles_m;
  const int tv = logical / tiles_m;
  const int m0 = tm * BM;
  const int v0 = tv * BV;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g = lane >> 4;

  // Every load below is unconditional: rows past V (or M) read the last valid
  // row and their outputs are never stored or ranked.  (Conditional loads
  // compile to branches whose joins drain the memory pipeline.)
  const graft_bf16 *wp[2];
#pragma unroll
  for (int vb = 0; vb < 2; ++vb) {
    const int r = v0 + wave * 32 + vb * 16 + l16;
    wp[vb] = w + static_cast<size_t>(r < V ? r : V - 1) * H + 8 * g;
  }
  // hidden staging: thread owns 16-byte column hcol of rows hrow0 + t * (kThreads / (KC / 8))
  constexpr int ROWS_PER_PASS = kThreads / (KC / 8);
  const int hcol = tid % (KC / 8);
  const int hrow0 = tid / (KC / 8);
  const graft_bf16 *hbase = hidden + hcol * 8;
  const int hd0 = hrow0 * STR + hcol * 8;

  f32x4 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 wa[2][KS], wb[2][KS], hr[PPT];
  auto load_w = [&](u32x4 (&d)[2][KS], int c) {
#pragma unroll
    for (int vb = 0; vb < 2; ++vb)
#pragma unroll
      for (int s = 0; s < KS; ++s)
        d[vb][s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wp[vb] + c * KC + s * 32));
  };
  auto load_h = [&](int c) {
#pragma unroll
    for (int t = 0; t < PPT; ++t) {
      const int m = min(m0 + hrow0 + t * ROWS_PER_PASS, M - 1);
      hr[t] = *reinterpret_cast<const u32x4 *>(hbase + static_cast<size_t>(m) * H + c * KC);
    }
  };
  auto store_h = [&](int buf) {
#pragma unroll
    for (int t = 0; t < PPT; ++t)
      *reinterpret_cast<u32x4 *>(&s_h[buf][hd0 + t * ROWS_PER_PASS * STR]) = hr[t];
  };
  auto compute = [&](const u32x4 (&d)[2][KS], int buf) {
    const graft_bf16 *hb = s_h[buf];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      bf16x8 bh[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        bh[mb] = *reinterpret_cast<const bf16x8 *>(&hb[(mb * 16 + l16) * STR + s * 32 + 8 * g]);
#pragma unroll
      for (int vb = 0; vb < 2; ++vb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          acc[vb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(d[vb][s]), bh[mb], acc[vb][mb], 0, 0, 0);
    }
  };

  // Two W register buffers used in strict ping-pong (the loop is unrolled by
  // two), so no register copy of an in-flight load ever forces a full wait.
  const int nch = H / KC;
  load_h(0);
  load_w(wa, 0);
  store_h(0);
  __syncthreads();
  for (int c = 0; c + 1 < nch; c += 2) {
    load_h(c + 1);
    load_w(wb, c + 1);
    __builtin_amdgcn_sched_barrier(0x38F);  // keep these loads ahead of the MFMAs
    compute(wa, 0);
    store_h(1);
    __syncthreads();
    const int c2 = c + 2 < nch ? c + 2 : c + 1;
    load_h(c2);
    load_w(wa, c2);
    __builtin_amdgcn_sched_barrier(0x38F);
    compute(wb, 1);
    store_h(0);
    __syncthreads();
  }
  if (nch & 1) {
    compute(wa, 0);
    __syncthreads();
  }

  // lane holds logit[m0 + mb*16 + l16][v0 + wave*32 + vb*16 + 4g + i]
  if constexpr (!FUSED) {
    const bool vec = (V & 3) == 0;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = m0 + mb * 16 + l16;
      if (m >= M) continue;
      float *row = logits + static_cast<size_t>(m) * V;
#pragma unroll
      for (int vb = 0; vb < 2; ++vb) {
        const int v = v0 + wave * 32 + vb * 16 + 4 * g;
        const f32x4 r = acc[vb][mb];
        if (vec && v < V) {
          *reinterpret_cast<float4 *>(row + v) = make_float4(r[0], r[1], r[2], r[3]);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (v + i < V) row[v + i] = r[i];
        }
      }
    }
  } else {
    float *s_t = reinterpret_cast<float *>(smem);
    // (the last barrier above ordered every read of s_h before this)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int vb = 0; vb < 2; ++vb) {
        const int vloc = wave * 32 + vb * 16 + 4 * g;
        *reinterpret_cast<f32x4 *>(&s_t[(mb * 16 + l16) * TSTR + vloc]) = acc[vb][mb];
      }
    __syncthreads();
    // WAVES consecutive threads per row, 32 entries each
    const int row = tid / WAVES;
    const int part = tid - row * WAVES;
    const int m = m0 + row;
    graft::TopKeys<K> L;
    L.init();
    const int vbase = v0 + part * 32;
#pragma unroll 8
    for (int j = 0; j < 32; ++j)
      if (vbase + j < V) L.insert(graft::rank_key(s_t[row * TSTR + part * 32 + j], vbase + j));
    for (int j = 0; j < k; ++j) {
      const uint64_t best = graft::group_max<WAVES>(L.k[0]);
      if (L.k[0] == best) L.pop_front();
      if (part == 0 && m < M) part_out[(static_cast<size_t>(m) * tiles_v + tv) * k + j] = best;
    }
  }
}

// ---------------------------------------------------------------- packed W
constexpr int PK_BV = 128;                  // vocabulary rows per tile
constexpr int PK_KC = 128;                  // hidden columns per chunk
constexpr int PK_NS = 3;                    // LDS ring stages
constexpr int PK_WB = PK_BV * PK_KC * 2;    // 32 KB of W per stage (two packed images)
constexpr int PK_IMG = PK_BV * 64 * 2;      // 16 KB packed image: 128 rows x 64 columns
constexpr int PK_HB = BM * PK_KC * 2;       // 16 KB hidden chunk
constexpr int PK_SB = PK_WB + PK_HB;        // one ring stage
constexpr int PK_GRID = 256;                // persistent workgroups (one per MI355X CU)
#ifndef GRAFT_PK_WAVES
#define GRAFT_PK_WAVES 8
#endif
constexpr int PK_WAVES = GRAFT_PK_WAVES;    // wavefronts per packed-path workgroup
constexpr int PK_TSTR = PK_BV + 4;          // floats per row of the staged logit tile
static_assert(BM * PK_TSTR * 4 <= PK_SB, "logit tile must fit in one ring stage");

// Image (tile t, column chunk j) at byte ((t * (H / 64) + j) * PK_IMG);
// inside it, byte r * 128 + p * 16 holds W[128 t + r][64 j + 8 p .. + 8],
// zero for rows >= V.  One thread per 16-byte piece.
__global__ __launch_bounds__(256) void lmhead_pack_kernel(int H, int V, const graft_bf16 *__restrict__ w,
                                                          u32x4 *__restrict__ out, size_t pieces) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= pieces) return;
  const int nkc = H / 64;
  const int p = static_cast<int>(i & 7);
  const int r = static_cast<int>((i >> 3) & (PK_BV - 1));
  const size_t img = i >> 10;  // 1024 pieces per image
  const int j = static_cast<int>(img % nkc);
  const size_t row = (img / nkc) * PK_BV + r;
  const int col = j * 64 + 8 * p;
  out[i] = row < static_cast<size_t>(V) ? *reinterpret_cast<const u32x4 *>(w + row * H + col) : zero4();
}

// 16-byte LDS DMA: lane l's 16 bytes from sbase + voff land at LDS byte
// lds + 16 l.  Issued through asm so the compiler does not serialise the
// ring with conservative waits; completion is tracked by hand with vmcnt.
__device__ inline void lds_dma16(unsigned lds, const void *sbase, unsigned voff) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(lds), "v"(voff), "s"(sbase)
               : "memory", "m0");
}
__device__ inline void lds_dma16_cached(unsigned lds, const void *sbase, unsigned voff) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(sbase)
               : "memory", "m0");
}
// Wait until at most N of this wave's DMAs are outstanding and every LDS
// access of this wave has completed, then meet the other waves.
template <int N>
__device__ inline void ring_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Which (m tile, tile stream) a persistent workgroup serves.  With T m-tiles
// and T <= 32, the 32 workgroups of one XCD (workgroups are dealt
// round-robin to the 8 XCDs) form 32/T groups of T: the T workgroups of a
// group take the same vocabulary tiles at the same time with different m
// tiles, so a W image fetched from HBM is re-read from that XCD's L2.
struct PkMap {
  int tm, stream, streams;
};
__device__ __host__ inline PkMap pk_map(int block, int T) {
  PkMap r;
  if (T <= 32) {
    const int groups = 32 / T;
    const int xcd = block % 8, slot = block / 8;
    const int gi = slot / T;
    r.tm = slot % T;
    r.streams = groups * 8;
    r.stream = gi < groups ? gi * 8 + xcd : -1;
  } else {
    r.streams = PK_GRID / T;
    r.tm = block % T;
    r.stream = block / T < r.streams ? block / T : -1;
  }
  return r;
}

// PW wavefronts per workgroup; wavefront w owns vocabulary rows
// [w * 128 / PW, (w + 1) * 128 / PW) of each tile and all 64 hidden rows.
// Larger per-wave tiles need fewer LDS fragment reads per MFMA (2 waves:
// 8 reads per 16 MFMAs; 4 waves: 6 per 8).
//
// SAMPLE (fused only): each row also draws a token at temperature T by the
// Gumbel-max identity, argmax_t fl(fl(l_t * inv_temp) + g_t) with the noise
// g read from `gumbel` [M, V]; one running best key per thread, one per
// (row, workgroup) into part_sample.  The noise loads are ordinary vector
// loads whose wait also covers the ring's older DMAs; they are issued before
// the tile's top-k work and consumed after it.
template <bool FUSED, int K, int PW, bool SAMPLE>
__global__ __launch_bounds__(PW * 64, 1) void lmhead_packed_kernel(int M, int H, int V, int k,
                                                                 const graft_bf16 *__restrict__ hidden,
                                                                 const unsigned char *__restrict__ wpk,
                                                                 float *__restrict__ logits,
                                                                 uint64_t *__restrict__ part_out, int tiles_m,
                                                                 int tiles_v, float inv_temp,
                                                                 const float *__restrict__ gumbel,
                                                                 uint64_t *__restrict__ part_sample) {
  static_assert(FUSED || !SAMPLE, "sampling rides on the fused epilogue");
  constexpr int NT = PW * 64;
  constexpr int VW = PK_BV / PW;      // vocabulary rows per wave
  constexpr int VBW = VW / 16;        // 16-row MFMA blocks per wave
  constexpr int WI = PK_WB / 1024 / PW;  // W DMA instructions per wave per stage
  constexpr int HI = PK_HB / 1024 / PW;  // hidden DMA instructions per wave per stage
  constexpr int TPR = NT / BM;        // epilogue threads per logit row
  constexpr int VPT = PK_BV / TPR;    // tile entries per epilogue thread
  constexpr int GPT = VPT / 8;        // groups of 8 entries per epilogue thread
  using PassT = typename std::conditional<(VPT > 32), uint64_t, uint32_t>::type;
  __shared__ __attribute__((aligned(1024))) unsigned char sm[PK_NS * PK_SB];
  const PkMap map = pk_map(blockIdx.x, tiles_m);
  if (map.stream < 0) return;
  const int S = map.streams;
  const int m0 = map.tm * BM;
  const int nch = H / PK_KC;
  const int items = map.stream < tiles_v ? (tiles_v - map.stream + S - 1) / S : 0;
  const int Q = items * nch;  // chunks this workgroup streams

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // LDS byte address of the ring (the M0 base of the DMAs)
  const unsigned sbase = static_cast<unsigned>(reinterpret_cast<size_t>((__attribute__((address_space(3))) void *)sm));

  // W images stream through L2 non-temporally unless several m tiles
  // (workgroups of one XCD) read each image
  const bool w_nt = tiles_m == 1;
  // loop-invariant DMA source offsets: each instruction fills four
  // 256-byte LDS rows, gathering their pieces from the chunk's two packed
  // images; hidden row r (clamped to M - 1) lands swizzled the same way
  unsigned wo[WI], ho[HI];
#pragma unroll
  for (int i = 0; i < WI; ++i) {
    // LDS row r holds logical piece p at slot p ^ (r & 15); pieces 0-7 come
    // from the chunk's first packed image, 8-15 from the second
    const int r = 4 * (wave * WI + i) + (lane >> 4);
    const int p = (lane & 15) ^ (r & 15);
    wo[i] = static_cast<unsigned>((p >> 3) * PK_IMG + r * 128 + (p & 7) * 16);
  }
#pragma unroll
  for (int i = 0; i < HI; ++i) {
    const int r = 4 * (wave * HI + i) + (lane >> 4);
    const int m = min(m0 + r, M - 1);
    ho[i] = static_cast<unsigned>(m) * H * 2 + (((lane & 15) ^ (r & 15)) * 16);
  }
  auto issue = [&](int q) {
    const int st = q % PK_NS;
    const int tv = map.stream + (q / nch) * S;
    const int c = q - (q / nch) * nch;
    const unsigned char *wsrc = wpk + (static_cast<size_t>(tv) * nch + c) * PK_WB;
    const unsigned char *hsrc = reinterpret_cast<const unsigned char *>(hidden) + c * PK_KC * 2;
    const unsigned wl = sbase + st * PK_SB + wave * WI * 1024;
    const unsigned hl = sbase + st * PK_SB + PK_WB + wave * HI * 1024;
#pragma unroll
    for (int i = 0; i < HI; ++i) lds_dma16_cached(hl + i * 1024, hsrc, ho[i]);
#pragma unroll
    for (int i = 0; i < WI; ++i) {
      if (w_nt) lds_dma16(wl + i * 1024, wsrc, wo[i]);
      else lds_dma16_cached(wl + i * 1024, wsrc, wo[i]);
    }
  };

  f32x4 acc[VBW][4];
#pragma unroll
  for (int a = 0; a < VBW; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  graft::TopKeys<K> L;
  L.init();
  uint64_t sbest = 0;  // SAMPLE: best perturbed key of this thread's entries

  if (Q > 0) issue(0);
  if (Q > 1) issue(1);
  for (int q = 0; q < Q; ++q) {
    // chunk q has landed once only chunk q + 1's DMAs may still be in flight
    if (q + 1 < Q) ring_barrier<WI + HI>();
    else ring_barrier<0>();
    if (q + 2 < Q) issue(q + 2);  // into the stage chunk q - 1 used
    const unsigned char *ws = sm + (q % PK_NS) * PK_SB;
    const unsigned char *hs = ws + PK_WB;
#pragma unroll
    for (int s = 0; s < PK_KC / 32; ++s) {
      const int P = s * 4 + g;  // 16-byte piece of the lane's 8 k values
      bf16x8 a[VBW], bh[4];
#pragma unroll
      for (int vb = 0; vb < VBW; ++vb)
        a[vb] = *reinterpret_cast<const bf16x8 *>(ws + (wave * VW + vb * 16 + l16) * 256 + (P ^ l16) * 16);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        bh[mb] = *reinterpret_cast<const bf16x8 *>(hs + (mb * 16 + l16) * 256 + (P ^ l16) * 16);
#pragma unroll
      for (int vb = 0; vb < VBW; ++vb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
          acc[vb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[vb], bh[mb], acc[vb][mb], 0, 0, 0);
    }
    if (q - (q / nch) * nch != nch - 1) continue;

    // ---- tile done: stage the 64 x 128 logits in this chunk's ring stage
    // (free until chunk q + 3 is issued, after the next ring barrier)
    const int v0 = (map.stream + (q / nch) * S) * PK_BV;
    float *s_t = reinterpret_cast<float *>(sm + (q % PK_NS) * PK_SB);
    __syncthreads();  // every wave is done reading the stage
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int vb = 0; vb < VBW; ++vb) {
        *reinterpret_cast<f32x4 *>(&s_t[(mb * 16 + l16) * PK_TSTR + wave * VW + vb * 16 + 4 * g]) = acc[vb][mb];
        acc[vb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    __syncthreads();
    if constexpr (FUSED) {
      // TPR consecutive threads per row, VPT entries each, into the
      // persistent lists.  Only entries that can still reach the row's top k
      // are inserted: an entry below the largest of the row's listed k-th
      // keys is beaten by k listed keys, and an entry below the k-th largest
      // of the tile row's 16 group maxima (groups of 8 entries) is beaten by
      // k entries of this tile.  The test is done on the float values (NaN
      // always passes, as its key ranks it); the insert compares keys.
      const int row = tid / TPR;
      const int part = tid - row * TPR;
      const int vb0 = v0 + part * VPT;
      const float *src = &s_t[row * PK_TSTR + part * VPT];
      float xv[VPT];
#pragma unroll
      for (int j4 = 0; j4 < VPT; j4 += 4) {
        const float4 x = *reinterpret_cast<const float4 *>(src + j4);
        xv[j4] = vb0 + j4 < V ? x.x : -INFINITY;
        xv[j4 + 1] = vb0 + j4 + 1 < V ? x.y : -INFINITY;
        xv[j4 + 2] = vb0 + j4 + 2 < V ? x.z : -INFINITY;
        xv[j4 + 3] = vb0 + j4 + 3 < V ? x.w : -INFINITY;
      }
      // SAMPLE: this row's noise is loaded first (16-byte loads while the
      // thread's 16 columns lie inside the row) and used only after the top-k
      // work below.  The wait for it also waits for the ring's two newest
      // chunks (the load counter is in order), once per tile: about 18 us of
      // the 22 the draw adds at 60 rows x 128256.  Columns past V re-read
      // column V - 1.
      float gv[SAMPLE ? VPT : 1];
      const int ms = m0 + row;
      if constexpr (SAMPLE) {
        const float *grow = gumbel + static_cast<size_t>(ms < M ? ms : M - 1) * V;
        if (vb0 + VPT <= V && (V & 3) == 0) {
#pragma unroll
          for (int j4 = 0; j4 < VPT; j4 += 4) {
            const float4 x = *reinterpret_cast<const float4 *>(grow + vb0 + j4);
            gv[j4] = x.x;
            gv[j4 + 1] = x.y;
            gv[j4 + 2] = x.z;
            gv[j4 + 3] = x.w;
          }
        } else {
#pragma unroll
          for (int j = 0; j < VPT; ++j) gv[j] = grow[min(vb0 + j, V - 1)];
        }
      }
      float gm[GPT];
#pragma unroll
      for (int q8 = 0; q8 < GPT; ++q8) {
        float m8 = xv[8 * q8];
#pragma unroll
        for (int e = 1; e < 8; ++e) m8 = fmaxf(m8, xv[8 * q8 + e]);
        gm[q8] = m8;
      }
      // k-th largest of the row's 16 maxima: k rounds of remove-the-largest
      // (equal maxima removed together only lower the bound, which keeps it
      // valid)
      float gk = -INFINITY;
      for (int r = 0; r < k; ++r) {
        float lm = gm[0];
#pragma unroll
        for (int q8 = 1; q8 < GPT; ++q8) lm = fmaxf(lm, gm[q8]);
        const float best = graft::group_maxf<TPR>(lm);
#pragma unroll
        for (int q8 = 0; q8 < GPT; ++q8) gm[q8] = gm[q8] == best ? -INFINITY : gm[q8];
        gk = best;
      }
      const uint64_t thr = graft::group_max<TPR>(L.k[K - 1]);
      const float tv = thr != 0 ? graft::key_value(thr) : -INFINITY;
      const float bound = fmaxf(gk, tv);
      PassT pass = 0;
#pragma unroll
      for (int j = 0; j < VPT; ++j) pass |= static_cast<PassT>(!(xv[j] < bound) & (vb0 + j < V)) << j;
      // entries re-read from LDS (no dynamic register indexing); the next
      // entry's read is issued before the current insert
      if (pass != 0) {
        int j = static_cast<int>(__builtin_ctzll(pass));
        float vj = src[j];
        while (true) {
          pass &= pass - 1;
          const int jn = pass != 0 ? static_cast<int>(__builtin_ctzll(pass)) : j;
          const float vn = src[jn];
          L.insert(graft::rank_key(vj, vb0 + j));
          if (pass == 0) break;
          j = jn;
          vj = vn;
        }
      }
      if constexpr (SAMPLE) {
        // two roundings, as defined: no fused multiply-add
#pragma clang fp contract(off)
        if (ms < M) {
#pragma unroll
          for (int j = 0; j < VPT; ++j) {
            if (vb0 + j < V) {
              const float scaled = xv[j] * inv_temp;
              float sc = scaled + gv[j];
              sc = sc != sc ? -INFINITY : sc;  // NaN ranks below every number
              const uint64_t key = graft::rank_key(sc, vb0 + j);
              sbest = key > sbest ? key : sbest;
            }
          }
        }
      }
    } else {
      // coalesced rows: 32 float4 per row
      const bool vec = (V & 3) == 0;
      for (int e = tid; e < BM * (PK_BV / 4); e += NT) {
        const int row = e / (PK_BV / 4);
        const int c4 = (e - row * (PK_BV / 4)) * 4;
        const int m = m0 + row;
        const int v = v0 + c4;
        if (m >= M || v >= V) continue;
        const float *src = &s_t[row * PK_TSTR + c4];
        float *dst = logits + static_cast<size_t>(m) * V + v;
        if (vec) {
          *reinterpret_cast<float4 *>(dst) = make_float4(src[0], src[1], src[2], src[3]);
        } else {
          for (int i = 0; i < 4 && v + i < V; ++i) dst[i] = src[i];
        }
      }
    }
  }
  if constexpr (FUSED) {
    // k best keys of each row over this workgroup's tiles (0 = no entry)
    const int row = tid / TPR;
    const int part = tid - row * TPR;
    const int m = m0 + row;
    for (int j = 0; j < k; ++j) {
      const uint64_t best = graft::group_max<TPR>(L.k[0]);
      if (L.k[0] == best) L.pop_front();
      if (part == 0 && m < M) part_out[(static_cast<size_t>(m) * S + map.stream) * k + j] = best;
    }
    if constexpr (SAMPLE) {
      const uint64_t best = graft::group_max<TPR>(sbest);
      if (part == 0 && m < M) part_sample[static_cast<size_t>(m) * S + map.stream] = best;
    }
  }
}

// ------------------------------------------------------ packed W, wide tiles
// Past 64 hidden rows the product leaves the HBM bound: at M = 960 it needs
// 0.49 ms of bf16 MFMA at the dense peak against 0.16 ms to stream W.  The
// 64-row kernel above would re-read every W image once per 64 rows, and its
// 16 x 64 wave tiles spend more LDS bandwidth than MFMA time.  Here a
// workgroup of 4 wavefronts computes a tile of 128 hidden rows x BV
// vocabulary rows, each wavefront a 64 x (BV / 2) block (2 x 2 layout), so
// one 16-byte fragment read feeds 8 / 3 MFMAs (BV = 256) and every byte a
// CU takes in feeds 85 flops.  That ratio is what bounds the kernel on
// MI355X: once HBM misses share a CU's request stream (and its in-order
// completion) the CU takes in about 30-35 GB/s, hits and misses alike.
//
// The ring stages 64 hidden columns at a time, one packed image per 128
// vocabulary rows (3 x 48 KB for BV = 256).  In LDS row r takes the 128
// bytes at r * 128 with its 16-byte pieces XOR-swizzled by (r % 8): the
// fragment reads measure 0.03 bank conflicts per access (rocprofv3
// LdsBankConflict; swapping the parity of rows r and r + 8 as well, which
// spreads 16 rows over all 64 banks on paper, measured 0.96).  Each DMA
// instruction fills eight rows of one image from 1 KB of contiguous
// source, so the image index is a scalar; the last tile's second image is
// clamped to the last image (its rows are all past V).
//
// Epilogue (per tile): the stage of the tile's last chunk is free until the
// next ring barrier; the 128 x BV logits go through it in 4 passes of 32
// rows.  8 threads per row screen BV / 8 entries each (interleaved 16-byte
// units, so the reads are conflict-free) into 4 persistent sorted lists per
// thread, one per pass; the bounds are those of the 64-row kernel.  One
// list per (row, workgroup) is written at the end, merged by
// topk_merge_kernel.  The k-order of the MFMA sums is that of every other
// path, so the logits are bit-identical.
constexpr int WD_BM = 128;  // hidden rows per tile
constexpr int WD_KC = 64;   // hidden columns per ring stage

__device__ inline const unsigned char *wd_uniform(const unsigned char *p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const unsigned char *>((static_cast<uint64_t>(hi) << 32) | lo);
}

// LDS byte offset of logical piece P (8 bf16) of row r in a stage region
__device__ inline int wd_piece(int r, int P) { return (r << 7) + ((P ^ (r & 7)) << 4); }

// Wait until at most n * D of this wave's DMAs are outstanding (n <= NMAX,
// picked at run time; vmcnt takes an immediate), then meet the other waves.
template <int D, int J, int NMAX>
__device__ inline void ring_barrier_n(int n) {
  static_assert(D * NMAX < 64, "vmcnt holds 6 bits");
  if constexpr (J >= NMAX) {
    ring_barrier<J * D>();
  } else {
    if (n == J) ring_barrier<J * D>();
    else ring_barrier_n<D, J + 1, NMAX>(n);
  }
}

template <int BV, int NS, int K>
__global__ __launch_bounds__(256, 1) void lmhead_wide_kernel(int M, int H, int V, int k,
                                                           const graft_bf16 *__restrict__ hidden,
                                                           const unsigned char *__restrict__ wpk,
                                                           uint64_t *__restrict__ part_out, int tiles_m,
                                                           int tiles_v, int n_img) {
  static_assert(BV == 128 || BV == 256, "one or two packed images per tile");
  constexpr int WB = BV * WD_KC * 2;     // W bytes per stage
  constexpr int HB = WD_BM * WD_KC * 2;  // hidden bytes per stage
  constexpr int SB = WB + HB;
  constexpr int WI = WB / 4096;          // W DMAs per wave per stage (1 KB each)
  constexpr int HI = HB / 4096;          // hidden DMAs per wave per stage
  constexpr int VW = BV / 2;             // vocabulary rows per wave
  constexpr int VB = VW / 16;            // 16-row MFMA blocks per wave
  constexpr int TSTR = BV + 4;           // floats per staged logit row
  constexpr int UPT = BV / 32;           // 16-byte units per screening thread
  constexpr int EPT = UPT * 4;           // entries per screening thread
  constexpr int GPT = EPT / 8;           // groups of 8 entries per thread
  static_assert(32 * TSTR * 4 <= SB, "32 staged logit rows must fit in one stage");
  static_assert(NS >= 3 && NS * SB <= 160 * 1024, "ring of 3+ stages in 160 KB of LDS");
  __shared__ __attribute__((aligned(1024))) unsigned char sm[NS * SB];

  const PkMap map = pk_map(blockIdx.x, tiles_m);
  if (map.stream < 0) return;
  const int S = map.streams;
  const int m0 = map.tm * WD_BM;
  const int nkc = H / WD_KC;
  const int items = map.stream < tiles_v ? (tiles_v - map.stream + S - 1) / S : 0;
  const int Q = items * nkc;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wv = wave & 1;
  const unsigned sbase = static_cast<unsigned>(reinterpret_cast<size_t>((__attribute__((address_space(3))) void *)sm));

  // DMA source offsets: lane -> (row, slot) -> logical piece -> its place
  // in the row-major packed image (W) or the row-major hidden state (rows
  // clamped to M - 1).
  unsigned wo[WI], ho[HI];
#pragma unroll
  for (int i = 0; i < WI; ++i) {
    const int r = 8 * (wave * WI + i) + (lane >> 3);
    const int P = (lane & 7) ^ (r & 7);
    wo[i] = static_cast<unsigned>((r & (PK_BV - 1)) * 128 + (P << 4));
  }
#pragma unroll
  for (int i = 0; i < HI; ++i) {
    const int r = 8 * (wave * HI + i) + (lane >> 3);
    const int P = (lane & 7) ^ (r & 7);
    const int m = min(m0 + r, M - 1);
    ho[i] = static_cast<unsigned>(m) * H * 2 + (P << 4);
  }
  // DMA issue, one instruction at a time: d < HI hidden, else W.  prep(q)
  // sets the scalar bases of stage q.
  const unsigned char *dw = wpk, *dh = reinterpret_cast<const unsigned char *>(hidden);
  unsigned dwl = sbase, dhl = sbase;
  auto prep = [&](int q) {
    const int st = q % NS;
    const int item = q / nkc;
    const int kc = q - item * nkc;
    const int tv = map.stream + item * S;
    const int img = min(tv * (BV / PK_BV) + (BV == 256 ? (wave >> 1) : 0), n_img - 1);
    dw = wd_uniform(wpk + (static_cast<size_t>(img) * nkc + kc) * PK_IMG);
    dh = wd_uniform(reinterpret_cast<const unsigned char *>(hidden) + kc * WD_KC * 2);
    dwl = sbase + st * SB + wave * WI * 1024;
    dhl = sbase + st * SB + WB + wave * HI * 1024;
  };
  auto dma = [&](auto d_tag) {
    constexpr int d = decltype(d_tag)::value;
    if constexpr (d < HI) lds_dma16_cached(dhl + d * 1024, dh, ho[d]);
    else lds_dma16_cached(dwl + (d - HI) * 1024, dw, wo[d - HI]);
  };

  // fragment offsets inside a stage (k-step s adds 4 to the logical piece)
  int fa[VB][2], fb[4][2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) fa[vb][s] = wd_piece(wv * VW + vb * 16 + l16, s * 4 + g);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) fb[mb][s] = WB + wd_piece(wm * 64 + mb * 16 + l16, s * 4 + g);
  }
  // 16-row blocks of this wave holding rows < M (wave-uniform)
  const int nmb = max(0, min(4, (M - m0 - wm * 64 + 15) >> 4));

  f32x4 acc[VB][4];
#pragma unroll
  for (int a = 0; a < VB; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  graft::TopKeys<K> lists[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) lists[p].init();

  const int srow = tid >> 3;  // screening: row srow of each 32-row pass
  const int part = tid & 7;

  constexpr int ND = WI + HI;  // DMAs per wave per stage
  // Software pipeline: the fragments of the next k-step are read while the
  // MFMAs of the current one run, and the next stage's DMAs are spread over
  // the first k-step's MFMA groups, so neither the LDS reads nor the
  // memory pipeline's back-pressure stall the MFMAs.  The ring barrier
  // sits between the two k-steps: it waits for stage q + 1 (and, for every
  // wave, the end of the reads of stage q), after which the first
  // fragments of stage q + 1 are read under the second k-step's MFMAs.
  auto load_frags = [&](const unsigned char *st, int s, bf16x8 (&a)[VB], bf16x8 (&b)[4]) {
#pragma unroll
    for (int vb = 0; vb < VB; ++vb) a[vb] = *reinterpret_cast<const bf16x8 *>(st + fa[vb][s]);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) b[mb] = *reinterpret_cast<const bf16x8 *>(st + fb[mb][s]);
  };
  auto mfma_vb = [&](int vb, const bf16x8 (&a)[VB], const bf16x8 (&b)[4]) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      acc[vb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[vb], b[mb], acc[vb][mb], 0, 0, 0);
  };
  // k-step 0 of a stage, with (ISS) the DMAs of the stage prep() chose
  auto kstep0 = [&](auto iss_tag, const bf16x8 (&a)[VB], const bf16x8 (&b)[4]) {
    constexpr bool ISS = decltype(iss_tag)::value;
    static_for<VB>([&](auto vb_tag) {
      constexpr int vb = decltype(vb_tag)::value;
      if constexpr (ISS) {
        static_for<(vb + 1) * ND / VB - vb * ND / VB>([&](auto j_tag) {
          dma(std::integral_constant<int, vb * ND / VB + decltype(j_tag)::value>{});
        });
      }
      mfma_vb(vb, a, b);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // a wave whose 64 rows all lie past M skips its MFMAs (uniform)
  const bool live = nmb > 0;

  bf16x8 a0[VB], b0[4], a1[VB], b1[4];
  for (int q = 0; q < NS - 1 && q < Q; ++q) {
    prep(q);
    static_for<ND>([&](auto d_tag) { dma(d_tag); });
  }
  if (Q > 0) {
    ring_barrier_n<ND, 0, NS - 2>(min(NS - 2, Q - 1));
    load_frags(sm, 0, a0, b0);
  }
  for (int q = 0; q < Q; ++q) {
    const unsigned char *st = sm + (q % NS) * SB;
    load_frags(st, 1, a1, b1);
    __builtin_amdgcn_sched_barrier(0);
    const bool iss = q + NS - 1 < Q;
    if (iss) prep(q + NS - 1);  // into the stage chunk q - 1 used
    if (live) {
      if (iss) kstep0(std::true_type{}, a0, b0);
      else kstep0(std::false_type{}, a0, b0);
    } else if (iss) {
      static_for<ND>([&](auto d_tag) { dma(d_tag); });
    }
    if (q + 1 < Q) {
      // stage q + 1 has landed once only the stages issued after it may be in flight
      ring_barrier_n<ND, 0, NS - 2>(min(NS - 2, Q - 2 - q));
      load_frags(sm + ((q + 1) % NS) * SB, 0, a0, b0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (live) {
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) mfma_vb(vb, a1, b1);
    }
    const int item = q / nkc;
    if (q - item * nkc != nkc - 1) continue;

    // ---- tile done
    const int v0 = (map.stream + item * S) * BV;
    float *s_t = reinterpret_cast<float *>(sm + (q % NS) * SB);
    __syncthreads();  // every wave is done reading the stage
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      if (wm == (p >> 1)) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int mb = 2 * (p & 1) + h;
#pragma unroll
          for (int vb = 0; vb < VB; ++vb)
            *reinterpret_cast<f32x4 *>(&s_t[(h * 16 + l16) * TSTR + wv * VW + vb * 16 + 4 * g]) = acc[vb][mb];
        }
      }
      __syncthreads();
      // unit u of this thread: 16-byte column 2 * part + (u & 1) + 16 * (u >> 1)
      const float *src = &s_t[srow * TSTR];
      float xv[EPT];
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        const int c = 4 * (2 * part + (u & 1) + 16 * (u >> 1));
        const float4 x = *reinterpret_cast<const float4 *>(src + c);
        xv[4 * u] = v0 + c < V ? x.x : -INFINITY;
        xv[4 * u + 1] = v0 + c + 1 < V ? x.y : -INFINITY;
        xv[4 * u + 2] = v0 + c + 2 < V ? x.z : -INFINITY;
        xv[4 * u + 3] = v0 + c + 3 < V ? x.w : -INFINITY;
      }
      // bound: the largest k-th key of the row's 8 lists; on the first tile
      // also the k-th largest of the row's group maxima (groups of 8 entries)
      const uint64_t thr = graft::group_max<8>(lists[p].k[K - 1]);
      float bound = thr != 0 ? graft::key_value(thr) : -INFINITY;
      if (item == 0) {
        float gm[GPT];
#pragma unroll
        for (int q8 = 0; q8 < GPT; ++q8) {
          float m8 = xv[8 * q8];
#pragma unroll
          for (int e = 1; e < 8; ++e) m8 = fmaxf(m8, xv[8 * q8 + e]);
          gm[q8] = m8;
        }
        float gk = -INFINITY;
        for (int r = 0; r < k; ++r) {
          float lm = gm[0];
#pragma unroll
          for (int q8 = 1; q8 < GPT; ++q8) lm = fmaxf(lm, gm[q8]);
          const float best = graft::group_maxf<8>(lm);
#pragma unroll
          for (int q8 = 0; q8 < GPT; ++q8) gm[q8] = gm[q8] == best ? -INFINITY : gm[q8];
          gk = best;
        }
        bound = fmaxf(bound, gk);
      }
      uint32_t pass = 0;
#pragma unroll
      for (int j = 0; j < EPT; ++j) pass |= static_cast<uint32_t>(!(xv[j] < bound)) << j;
      if (m0 + 32 * p + srow >= M) pass = 0;
      while (pass != 0) {
        const int j = __builtin_ctz(pass);
        pass &= pass - 1;
        const int c = 4 * (2 * part + ((j >> 2) & 1) + 16 * (j >> 3)) + (j & 3);
        if (v0 + c < V) lists[p].insert(graft::rank_key(src[c], v0 + c));
      }
      __syncthreads();  // the next pass overwrites the staged rows
    }
#pragma unroll
    for (int a = 0; a < VB; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // k best keys of each row over this workgroup's tiles (0 = no entry)
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int m = m0 + 32 * p + srow;
    for (int j = 0; j < k; ++j) {
      const uint64_t best = graft::group_max<8>(lists[p].k[0]);
      if (lists[p].k[0] == best) lists[p].pop_front();
      if (part == 0 && m < M) part_out[(static_cast<size_t>(m) * S + map.stream) * k + j] = best;
    }
  }
}


// ------------------------------------------------ packed W, 256 x 256 tiles
// Past 128 hidden rows every byte a CU takes in is worth more flops with a
// bigger tile: a 256 x 256 tile (hidden rows x vocabulary rows) feeds 128
// flops per byte taken in against the 128 x 256 tile's 85.  4 wavefronts,
// each a 128 x 128 block (2 x 2 layout): 64 accumulator tiles (256
// accumulation registers) and 8 + 8 fragments per k-step, read as in the
// 128-row kernel from 128-byte LDS rows swizzled by (r % 8).
//
// A chunk is 64 hidden columns: 32 KB of W (two packed images) and 32 KB of
// hidden rows.  W goes through a ring of three stages and the hidden rows
// through a ring of two (160 KB in all).  What bounds the loop besides the
// MFMAs is the number of copy instructions, not their bytes: copies of 4
// bytes per lane instead of 16 take as long, and the copies cost about a
// fifth of the kernel's time even when no wait for them remains, so they
// are issued one per group of 8 MFMAs, never in bursts (the schedule is
// described at the ring below).
//
// Epilogue (per tile): one thread per hidden row keeps one persistent sorted
// list of k keys.  The tile's logits pass through the chunk's two consumed
// stages (rows 0-127 in its W stage, 128-255 in its hidden stage) in 8
// passes of 32 vocabulary columns; each thread screens its row's 32 entries
// against its own k-th key.  One list per (row, workgroup) is written at the
// end and merged by topk_merge_kernel.  The MFMA sums run in the k-order of
// every other path, so the logits are bit-identical.
using graft::F64Keys;

constexpr int BG_BM = 256;  // hidden rows per tile
constexpr int BG_BV = 256;  // vocabulary rows per tile

template <int K>
__global__ __launch_bounds__(256, 1) void lmhead_big_kernel(int M, int H, int V, int k,
                                                          const graft_bf16 *__restrict__ hidden,
                                                          const unsigned char *__restrict__ wpk,
                                                          uint64_t *__restrict__ part_out, int tiles_m, int tiles_v,
                                                          int n_img) {
  constexpr int WB = BG_BV * WD_KC * 2;  // W bytes per chunk (two packed images)
  constexpr int HB = BG_BM * WD_KC * 2;  // hidden bytes per chunk
  constexpr int NW = 3, NH = 2;          // ring stages
  constexpr int WI = WB / 4096;          // W DMAs per wave per chunk (1 KB each)
  constexpr int HI = HB / 4096;          // hidden DMAs per wave per chunk
  constexpr int VB = 8;                  // 16-row vocabulary blocks per wave
  constexpr int MB = 8;                  // 16-row hidden blocks per wave
  constexpr int CW = 32;                 // vocabulary columns per epilogue pass
  constexpr int TSTR = CW + 4;           // floats per staged logit row
  static_assert(128 * TSTR * 4 <= WB && 128 * TSTR * 4 <= HB, "half a pass fits in a stage");
  static_assert(WI == VB && HI == VB && MB == VB, "two fragment reads and one DMA per MFMA group");
  static_assert(NW * WB + NH * HB <= 160 * 1024, "the rings fit in 160 KB of LDS");
  __shared__ __attribute__((aligned(1024))) unsigned char sm[NW * WB + NH * HB];
  unsigned char *const sw = sm;
  unsigned char *const sh = sm + NW * WB;

  const PkMap map = pk_map(blockIdx.x, tiles_m);
  if (map.stream < 0) return;
  const int S = map.streams;
  const int m0 = map.tm * BG_BM;
  const int nkc = H / WD_KC;
  const int items = map.stream < tiles_v ? (tiles_v - map.stream + S - 1) / S : 0;
  const int Q = items * nkc;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wv = wave & 1;
  const unsigned sbase = static_cast<unsigned>(reinterpret_cast<size_t>((__attribute__((address_space(3))) void *)sm));

  // DMA source offsets: lane -> (row, slot) -> logical piece -> its place in
  // the row-major packed image (W; waves 0-1 fill the first image's 128
  // rows, waves 2-3 the second's) or the row-major hidden state (rows
  // clamped to M - 1)
  unsigned wo[WI], ho[HI];
#pragma unroll
  for (int i = 0; i < WI; ++i) {
    const int r = 8 * (wave * WI + i) + (lane >> 3);
    const int P = (lane & 7) ^ (r & 7);
    wo[i] = static_cast<unsigned>((r & (PK_BV - 1)) * 128 + (P << 4));
  }
#pragma unroll
  for (int i = 0; i < HI; ++i) {
    const int r = 8 * (wave * HI + i) + (lane >> 3);
    const int P = (lane & 7) ^ (r & 7);
    const int m = min(m0 + r, M - 1);
    ho[i] = static_cast<unsigned>(m) * H * 2 + (P << 4);
  }
  // Sources and LDS targets of chunk j's W (W stage j % 3) and hidden rows
  // (hidden stage j % 2).  A chunk past the last one (j >= Q) re-reads the
  // last chunk into the stage it would use, which nothing reads again: the
  // DMAs then need no branch, and the waits below stay the same every chunk.
  struct Dma {
    const unsigned char *src;
    unsigned dst;
  };
  auto w_dma = [&](int j) {
    const int jj = min(j, Q - 1);
    const int item = jj / nkc;
    const int kc = jj - item * nkc;
    const int tv = map.stream + item * S;
    const int img = min(tv * 2 + (wave >> 1), n_img - 1);
    return Dma{wd_uniform(wpk + (static_cast<size_t>(img) * nkc + kc) * PK_IMG),
               sbase + (j % NW) * WB + wave * WI * 1024};
  };
  auto h_dma = [&](int j) {
    const int jj = min(j, Q - 1);
    const int kc = jj - (jj / nkc) * nkc;
    return Dma{wd_uniform(reinterpret_cast<const unsigned char *>(hidden) + kc * WD_KC * 2),
               sbase + NW * WB + (j % NH) * HB + wave * HI * 1024};
  };

  // fragment offsets inside a stage: the swizzle depends on l16 only, so
  // block b adds b * 16 rows of 128 bytes
  int fa[2], fb[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    fa[s] = wd_piece(wv * 128 + l16, s * 4 + g);
    fb[s] = wd_piece(wm * 128 + l16, s * 4 + g);
  }
  // (a wave whose rows all lie past M still runs its MFMAs, on the clamped
  // rows; their logits are never screened)
  F64Keys<K> list;  // hidden row m0 + tid
  list.init();

  // Ring schedule.  Chunk j's W sits in W stage j % 3 and its hidden rows in
  // hidden stage j % 2.  The chunk's one barrier, B_j, sits between its two
  // k-steps: the second k-step's fragments are read during the first, so
  // at B_j every wave holds them in registers (chunk j's stages are no
  // longer read) and no MFMA after the barrier waits on LDS; B_j also makes
  // sure chunk j + 1 has landed.  The DMAs go eight per k-step, one per
  // group of 8 MFMAs: W_j+2 in chunk j's first k-step (into the stage chunk
  // j - 1 left at B_j-1), H_j+2 in its second (into chunk j's own hidden
  // stage); both must land by B_j+1.  (Issued evenly over both k-steps
  // instead of sixteen in one, and with the barrier here instead of at the
  // chunk's top, the kernel measured about 5% faster.)  A tile's last chunk
  // leaves its stages to the epilogue, which stages the tile's logits there
  // and then issues that chunk's H_j+2.
  //
  // Prologue, in the order the waits assume: W_0, H_0, W_1, H_1; the first
  // chunk's data must land before anything is read.
  if (Q > 0) {
    const Dma w0 = w_dma(0), h0 = h_dma(0), w1 = w_dma(1), h1 = h_dma(1);
#pragma unroll
    for (int i = 0; i < WI; ++i) lds_dma16_cached(w0.dst + i * 1024, w0.src, wo[i]);
#pragma unroll
    for (int i = 0; i < HI; ++i) lds_dma16_cached(h0.dst + i * 1024, h0.src, ho[i]);
#pragma unroll
    for (int i = 0; i < WI; ++i) lds_dma16_cached(w1.dst + i * 1024, w1.src, wo[i]);
#pragma unroll
    for (int i = 0; i < HI; ++i) lds_dma16_cached(h1.dst + i * 1024, h1.src, ho[i]);
    ring_barrier<WI + HI>();  // W_0 and H_0 have landed, for every wave
  }
  auto fw = [&](int j, int off) {
    return *reinterpret_cast<const bf16x8 *>(sw + (j % NW) * WB + off);
  };
  auto fh = [&](int j, int off) {
    return *reinterpret_cast<const bf16x8 *>(sh + (j % NH) * HB + off);
  };
  // fragments of the k-step in use (a: vocabulary, b: hidden) and of the
  // next one, being read
  bf16x8 a0[VB], b0[MB], a1[VB], b1[MB];
  int q = 0;
  for (int item = 0; item < items; ++item) {
    f32x4 acc[VB][MB];
#pragma unroll
    for (int a = 0; a < VB; ++a)
#pragma unroll
      for (int b = 0; b < MB; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    // One chunk, both k-steps in one straight run (code paths that branch
    // between MFMA groups make the register allocator move the 256
    // accumulators at every block edge; for the same reason no fragment is
    // carried from one chunk to the next).  The first k-step's fragments
    // are read at the top, in the order its first groups use them; in each
    // group of the first k-step two fragments of the second are read (the
    // hidden ones first: every group needs all of them).
    auto chunk = [&](auto last_tag, int j) {
      constexpr bool LAST = decltype(last_tag)::value;
      a0[0] = fw(j, fa[0]);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) b0[mb] = fh(j, fb[0] + mb * 2048);
#pragma unroll
      for (int vb = 1; vb < VB; ++vb) a0[vb] = fw(j, fa[0] + vb * 2048);
      __builtin_amdgcn_sched_barrier(0);
      const Dma wn = w_dma(j + 2);
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) {
        if (vb < VB / 2) {
          b1[2 * vb] = fh(j, fb[1] + 2 * vb * 2048);
          b1[2 * vb + 1] = fh(j, fb[1] + (2 * vb + 1) * 2048);
        } else {
          a1[2 * vb - VB] = fw(j, fa[1] + (2 * vb - VB) * 2048);
          a1[2 * vb - VB + 1] = fw(j, fa[1] + (2 * vb - VB + 1) * 2048);
        }
        lds_dma16_cached(wn.dst + vb * 1024, wn.src, wo[vb]);
        __builtin_amdgcn_sched_barrier(0);  // the reads stay ahead of these MFMAs
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[vb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[vb], b0[mb], acc[vb][mb], 0, 0, 0);
      }
      // B_j: this wave's reads of chunk j are done and, with W_j+2 (the
      // youngest DMAs) still allowed in flight, W_j+1 and H_j+1 have landed
      ring_barrier<WI>();
      Dma hn{nullptr, 0u};
      if constexpr (!LAST) hn = h_dma(j + 2);
#pragma unroll
      for (int vb = 0; vb < VB; ++vb) {
        if constexpr (!LAST) lds_dma16_cached(hn.dst + vb * 1024, hn.src, ho[vb]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[vb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[vb], b1[mb], acc[vb][mb], 0, 0, 0);
      }
    };
    for (int kc = 0; kc + 1 < nkc; ++kc, ++q) chunk(std::false_type{}, q);
    chunk(std::true_type{}, q);
    ++q;

    // ---- tile done: its logits go through the last chunk's two stages
    // (rows 0-127 in the W stage, 128-255 in the hidden stage) in passes of
    // 32 vocabulary columns
    const int v0 = (map.stream + item * S) * BG_BV;
    float *s_w = reinterpret_cast<float *>(sw + ((q - 1) % NW) * WB);
    float *s_h = reinterpret_cast<float *>(sh + ((q - 1) % NH) * HB);
    float *s_wave = wm == 0 ? s_w : s_h;  // this wave's rows
    const float *src = (tid < 128 ? s_w : s_h) + (tid & 127) * TSTR;
    const bool row_ok = m0 + tid < M;
    __syncthreads();  // every wave is done reading the stages
#pragma unroll
    for (int p = 0; p < BG_BV / CW; ++p) {
      if (wv == (p >> 2)) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int vb = 2 * (p & 3) + h;
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) {
            // stored straight from the accumulation registers ("a")
            const unsigned addr = static_cast<unsigned>(reinterpret_cast<size_t>(
                (__attribute__((address_space(3))) float *)&s_wave[(mb * 16 + l16) * TSTR + h * 16 + 4 * g]));
            asm volatile("ds_write_b128 %0, %1" ::"v"(addr), "a"(acc[vb][mb]) : "memory");
          }
        }
        // the compiler does not count the asm stores: wait for them here
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
      __syncthreads();
      // Screening: a candidate bit per entry at least the row's k-th key
      // value; in the workgroup's first pass, while the lists are still
      // empty, also at least the k-th largest of the pass's group maxima
      // (K groups of CW / K entries: K entries of the pass are at least that
      // large, so a smaller entry is not in the top k; with k < K the bound
      // is lower than needed, still valid).  After that pass every list is
      // full.  Columns past V (zero rows of the last tile) never count.  The
      // inserts then run once per candidate of the lane with the most, not
      // once per entry that any lane keeps.
      const int c0 = v0 + p * CW;
      uint32_t cand = 0;
      auto screen = [&](auto first_tag, auto tail_tag) {
        constexpr bool FIRST = decltype(first_tag)::value;
        constexpr bool TAIL = decltype(tail_tag)::value;
        float xv[CW];
#pragma unroll
        for (int u = 0; u < CW / 4; ++u) {
          const float4 x = *reinterpret_cast<const float4 *>(src + 4 * u);
          xv[4 * u] = x.x;
          xv[4 * u + 1] = x.y;
          xv[4 * u + 2] = x.z;
          xv[4 * u + 3] = x.w;
        }
        if constexpr (TAIL) {
#pragma unroll
          for (int e = 0; e < CW; ++e) xv[e] = c0 + e < V ? xv[e] : -INFINITY;
        }
        float bound = list.kth_value();
        if constexpr (FIRST) {
          constexpr int GS = CW / K;  // entries per group (4 for k <= 8 lists, 2 for 16)
          float gmin = INFINITY;
#pragma unroll
          for (int gi = 0; gi < K; ++gi) {
            float gm = xv[gi * GS];
#pragma unroll
            for (int e = 1; e < GS; ++e) gm = fmaxf(gm, xv[gi * GS + e]);
            gmin = fminf(gmin, gm);
          }
          if (k == K) bound = fmaxf(bound, gmin);
        }
#pragma unroll
        for (int e = 0; e < CW; ++e) {
          bool keep = !(xv[e] < bound);
          if constexpr (TAIL) keep = keep && c0 + e < V;
          cand |= static_cast<uint32_t>(keep) << e;
        }
      };
      const bool first = item == 0 && p == 0;  // uniform
      const bool tail = v0 + BG_BV > V;         // uniform
      if (first) {
        if (tail) screen(std::true_type{}, std::true_type{});
        else screen(std::true_type{}, std::false_type{});
      } else {
        if (tail) screen(std::false_type{}, std::true_type{});
        else screen(std::false_type{}, std::false_type{});
      }
      if (!row_ok) cand = 0;
      // as many rounds as the lane with the most candidates, every lane in
      // every round (a lane with none left inserts the empty key): no
      // divergent branches
      const uint32_t rounds = graft::wave_max_u32(static_cast<uint32_t>(__popc(cand)));
      for (uint32_t r = 0; r < rounds; ++r) {
        const int j = cand != 0 ? __builtin_ctz(cand) : 0;
        const double key = cand != 0 ? F64Keys<K>::make(src[j], c0 + j) : 0.0;
        cand &= cand - 1;
        list.insert(key);
      }
      __syncthreads();  // the next pass overwrites the staged rows
    }
    // the staging stages are free again: the hidden rows two chunks after
    // the tile's last one (q - 1) go into its hidden stage (W of the chunk
    // after them goes into its W stage during the next chunk)
    if (item + 1 < items) {
      const Dma hn = h_dma(q + 1);
#pragma unroll
      for (int i = 0; i < HI; ++i) lds_dma16_cached(hn.dst + i * 1024, hn.src, ho[i]);
    }
  }
  // the DMAs past the last chunk must land before the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // this workgroup's k best keys of row m0 + tid (0 = no entry)
  const int m = m0 + tid;
  if (m < M) {
    uint64_t *dst = part_out + (static_cast<size_t>(m) * S + map.stream) * k;
#pragma unroll
    for (int j = 0; j < K; ++j)
      if (j < k) dst[j] = list.rank_key(j);
  }
}

}  // namespace

namespace graft {
size_t lmhead_fused_ws_bytes(int M, int V, int k) {
  const int tiles_v = (V + kBV - 1) / kBV;
  return static_cast<size_t>(M) * tiles_v * k * sizeof(uint64_t);
}
}  // namespace graft

namespace {
int packed_tiles_m(int M) { return (M + BM - 1) / BM; }
int wide_tiles_m(int M) { return (M + WD_BM - 1) / WD_BM; }
int big_tiles_m(int M) { return (M + BG_BM - 1) / BG_BM; }
// Above 128 rows the 256 x 256 tiles (128 flops per byte taken in).
bool packed_big(int M) { return M > WD_BM; }
// The fused packed path takes the wide tiles above 64 rows (65-128 rows:
// one m tile, each W image read once; the 64-row kernel would run two m
// tiles sharing each image through L2, about 3% slower).  Up to 64 rows
// the 64-row kernel's 8 wavefronts stream W faster than 4.
bool packed_wide(int M) { return M > BM; }
size_t packed_fused_ws_bytes(int M, int k) {
  const int T = packed_big(M) ? big_tiles_m(M) : (packed_wide(M) ? wide_tiles_m(M) : packed_tiles_m(M));
  if (packed_tiles_m(M) > PK_GRID) return 0;
  return static_cast<size_t>(M) * pk_map(0, T).streams * k * sizeof(uint64_t);
}
}  // namespace

extern "C" size_t graft_lmhead_pack_bytes(int V, int H) {
  if (V <= 0 || H <= 0 || H % PK_KC != 0) return 0;
  return static_cast<size_t>((V + PK_BV - 1) / PK_BV) * PK_BV * H * 2;
}

extern "C" int graft_lmhead_pack(int V, int H, const graft_bf16 *w, graft_bf16 *w_packed, graft_stream stream) {
  using graft::fail;
  if (V <= 0 || H <= 0 || H % PK_KC != 0)
    return fail(GRAFT_EINVAL, "lmhead_pack: V=%d H=%d (H must be a positive multiple of %d)", V, H, PK_KC);
  if (!w || !w_packed) return fail(GRAFT_EINVAL, "lmhead_pack: NULL array");
  if (!graft::aligned16(w) || !graft::aligned16(w_packed))
    return fail(GRAFT_EINVAL, "lmhead_pack: w and w_packed must be 16-byte aligned");
  graft::clear_error();
  const size_t pieces = graft_lmhead_pack_bytes(V, H) / 16;
  const size_t blocks = (pieces + 255) / 256;
  if (blocks > 0x7FFFFFFFull) return fail(GRAFT_EINVAL, "lmhead_pack: too large");
  hipLaunchKernelGGL(lmhead_pack_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, graft::as_stream(stream), H, V,
                     w, reinterpret_cast<u32x4 *>(w_packed), pieces);
  return graft::check_launch("lmhead_pack");
}

extern "C" size_t graft_lmhead_topk_workspace_bytes(int M, int V, int k) {
  if (M <= 0 || V <= 0 || k <= 0) return 0;
  size_t a = graft::topk_plan(M, V, k).ws_bytes;
  const size_t b = graft::lmhead_fused_ws_bytes(M, V, k);
  const size_t c = packed_fused_ws_bytes(M, k);
  if (b > a) a = b;
  return c > a ? c : a;
}

extern "C" int graft_lmhead_topk(int M, int H, int V, int k, const graft_bf16 *hidden, const graft_bf16 *w,
                                 int w_layout, float *logits, int32_t *topk_id, float *topk_val, void *ws,
                                 size_t ws_bytes, graft_stream stream) {
  using graft::fail;
  if (M < 0 || V <= 0 || V > GRAFT_MAX_V || k < 0 || k > GRAFT_MAX_K || k > V)
    return fail(GRAFT_EINVAL, "lmhead_topk: M=%d V=%d k=%d", M, V, k);
  if (w_layout != GRAFT_W_ROWMAJOR && w_layout != GRAFT_W_PACKED)
    return fail(GRAFT_EINVAL, "lmhead_topk: unknown weight layout %d", w_layout);
  const bool packed = w_layout == GRAFT_W_PACKED;
  if (hidden && (H <= 0 || H % (packed ? PK_KC : 64) != 0))
    return fail(GRAFT_EINVAL, "lmhead_topk: H=%d must be a positive multiple of %d", H, packed ? PK_KC : 64);
  if (!hidden && !logits) return fail(GRAFT_EINVAL, "lmhead_topk: both hidden and logits are NULL");
  if (hidden && !w) return fail(GRAFT_EINVAL, "lmhead_topk: W is NULL");
  if (!logits && k == 0) return fail(GRAFT_EINVAL, "lmhead_topk: fused mode needs k > 0");
  if (!hidden && k == 0) return fail(GRAFT_EINVAL, "lmhead_topk: nothing to do (no hidden, k = 0)");
  if (k > 0 && !topk_id) return fail(GRAFT_EINVAL, "lmhead_topk: topk_id is NULL");
  if (hidden && packed && packed_tiles_m(M) > PK_GRID)
    return fail(GRAFT_EINVAL, "lmhead_topk: M=%d exceeds the packed path's %d rows", M, PK_GRID * BM);
  if (hidden && packed && static_cast<size_t>(M) * H * 2 > 0xFFFFFFFFull)
    return fail(GRAFT_EINVAL, "lmhead_topk: hidden of %d x %d exceeds 4 GiB (32-bit DMA offsets)", M, H);
  if (M == 0) return GRAFT_OK;
  if ((hidden && !graft::aligned16(hidden)) || (hidden && !graft::aligned16(w)) || (logits && !graft::aligned16(logits)))
    return fail(GRAFT_EINVAL, "lmhead_topk: hidden, w and logits must be 16-byte aligned");
  const bool fused = hidden && !logits;
  size_t need = k > 0 && !fused ? graft::topk_plan(M, V, k).ws_bytes : 0;
  if (fused) need = packed ? packed_fused_ws_bytes(M, k) : graft::lmhead_fused_ws_bytes(M, V, k);
  if (ws_bytes < need || (need > 0 && !ws))
    return fail(GRAFT_EINVAL, "lmhead_topk: workspace %zu bytes < %zu", ws_bytes, need);
  graft::clear_error();
  hipStream_t s = graft::as_stream(stream);
  using I64 = std::integral_constant<int, 64>;
  using I128 = std::integral_constant<int, 128>;
  using I8 = std::integral_constant<int, 8>;
  using I16 = std::integral_constant<int, 16>;
  using T = std::true_type;
  using Fz = std::false_type;

  if (hidden && packed) {
    const int tiles_m = packed_tiles_m(M);
    const int tiles_v = (V + PK_BV - 1) / PK_BV;
    const unsigned char *wpk = reinterpret_cast<const unsigned char *>(w);
    auto launch = [&](auto fused_tag, auto k_tag, uint64_t *pk) {
      constexpr bool F = decltype(fused_tag)::value;
      constexpr int Kv = decltype(k_tag)::value;
      hipLaunchKernelGGL((lmhead_packed_kernel<F, Kv, PK_WAVES, false>), dim3(PK_GRID), dim3(PK_WAVES * 64), 0, s, M, H, V,
                         F ? k : 0, hidden, wpk, F ? nullptr : logits, pk, tiles_m, tiles_v, 1.0f, nullptr, nullptr);
    };
    if (fused && packed_big(M)) {
      uint64_t *pk = static_cast<uint64_t *>(ws);
      const int Tb = big_tiles_m(M);
      const int n_img = (V + PK_BV - 1) / PK_BV;
      const int tv = (V + BG_BV - 1) / BG_BV;
      if (k <= 8)
        hipLaunchKernelGGL((lmhead_big_kernel<8>), dim3(PK_GRID), dim3(256), 0, s, M, H, V, k, hidden, wpk, pk, Tb, tv,
                           n_img);
      else
        hipLaunchKernelGGL((lmhead_big_kernel<16>), dim3(PK_GRID), dim3(256), 0, s, M, H, V, k, hidden, wpk, pk, Tb,
                           tv, n_img);
      int rc = graft::check_launch("lmhead (packed, 256 x 256 tiles, fused top-k)");
      if (rc != GRAFT_OK) return rc;
      return graft::launch_topk_merge(M, pk_map(0, Tb).streams, k, pk, topk_id, topk_val, s);
    }
    if (fused && packed_wide(M)) {
      uint64_t *pk = static_cast<uint64_t *>(ws);
      const int Tw = wide_tiles_m(M);
      const int n_img = (V + PK_BV - 1) / PK_BV;
      auto launch_w = [&](auto bv_tag, auto k_tag) {
        constexpr int BVv = decltype(bv_tag)::value;
        constexpr int Kv = decltype(k_tag)::value;
        constexpr int NSv = BVv == 256 ? 3 : 4;
        const int tv = (V + BVv - 1) / BVv;
        hipLaunchKernelGGL((lmhead_wide_kernel<BVv, NSv, Kv>), dim3(PK_GRID), dim3(256), 0, s, M, H, V, k, hidden, wpk,
                           pk, Tw, tv, n_img);
      };
      using I256 = std::integral_constant<int, 256>;
      // (two images with 16-key lists would spill registers)
      if (k <= 8) launch_w(I256{}, I8{});
      else launch_w(I128{}, I16{});
      int rc = graft::check_launch("lmhead (packed, wide tiles, fused top-k)");
      if (rc != GRAFT_OK) return rc;
      return graft::launch_topk_merge(M, pk_map(0, Tw).streams, k, pk, topk_id, topk_val, s);
    }
    if (fused) {
      uint64_t *pk = static_cast<uint64_t *>(ws);
      if (k <= 8) launch(T{}, I8{}, pk);
      else launch(T{}, I16{}, pk);
      int rc = graft::check_launch("lmhead (packed, fused top-k)");
      if (rc != GRAFT_OK) return rc;
      return graft::launch_topk_merge(M, pk_map(0, tiles_m).streams, k, pk, topk_id, topk_val, s);
    }
    launch(Fz{}, I8{}, nullptr);
    int rc = graft::check_launch("lmhead (packed)");
    if (rc != GRAFT_OK) return rc;
    if (k > 0) return graft::launch_topk(M, V, k, logits, topk_id, topk_val, ws, s);
    return GRAFT_OK;
  }

  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_v = (V + kBV - 1) / kBV;
  const int grid = (tiles_m * tiles_v + 7) / 8 * 8;
  // K chunk of 128 hidden columns when it divides H (the common case), else 64
  const bool kc128 = H % 128 == 0;
  auto launch = [&](auto kc_tag, auto fused_tag, auto k_tag, uint64_t *pk) {
    constexpr int KCv = decltype(kc_tag)::value;
    constexpr bool F = decltype(fused_tag)::value;
    constexpr int Kv = decltype(k_tag)::value;
    hipLaunchKernelGGL((lmhead_kernel<KCv, F, Kv>), dim3(grid), dim3(kThreads), 0, s, M, H, V, F ? k : 0, hidden, w,
                       F ? nullptr : logits, pk, tiles_m, tiles_v);
  };
  if (fused) {
    uint64_t *pk = static_cast<uint64_t *>(ws);
    if (kc128 && k <= 8) launch(I128{}, T{}, I8{}, pk);
    else if (kc128) launch(I128{}, T{}, I16{}, pk);
    else if (k <= 8) launch(I64{}, T{}, I8{}, pk);
    else launch(I64{}, T{}, I16{}, pk);
    int rc = graft::check_launch("lmhead (fused top-k)");
    if (rc != GRAFT_OK) return rc;
    return graft::launch_topk_merge(M, tiles_v, k, pk, topk_id, topk_val, s);
  }
  if (hidden) {
    if (kc128) launch(I128{}, Fz{}, I8{}, nullptr);
    else launch(I64{}, Fz{}, I8{}, nullptr);
    int rc = graft::check_launch("lmhead");
    if (rc != GRAFT_OK) return rc;
  }
  if (k > 0) return graft::launch_topk(M, V, k, logits, topk_id, topk_val, ws, s);
  return GRAFT_OK;
}

namespace {
size_t packed_sample_ws_bytes(int M, int k) {
  const int T = packed_tiles_m(M);
  if (T > PK_GRID) return 0;
  const size_t S = static_cast<size_t>(pk_map(0, T).streams);
  const size_t topk = static_cast<size_t>(M) * S * k * sizeof(uint64_t);
  const size_t samp = static_cast<size_t>(M) * S * sizeof(uint64_t);
  return topk + samp;
}
}  // namespace

extern "C" size_t graft_lmhead_sample_workspace_bytes(int M, int V, int k) {
  if (M <= 0 || V <= 0 || k <= 0 || k > GRAFT_MAX_K) return 0;
  return packed_sample_ws_bytes(M, k);
}

extern "C" int graft_lmhead_topk_sample(int M, int H, int V, int k, float temperature, const graft_bf16 *hidden,
                                        const graft_bf16 *w_packed, const float *gumbel, int32_t *topk_id,
                                        float *topk_val, int32_t *sample_id, void *ws, size_t ws_bytes,
                                        graft_stream stream) {
  using graft::fail;
  if (M < 0 || V <= 0 || k < 1 || k > GRAFT_MAX_K || k > V)
    return fail(GRAFT_EINVAL, "lmhead_topk_sample: M=%d V=%d k=%d", M, V, k);
  if (!(temperature > 0.f) || !(temperature < INFINITY))
    return fail(GRAFT_EINVAL, "lmhead_topk_sample: temperature must be positive and finite");
  if (H <= 0 || H % PK_KC != 0)
    return fail(GRAFT_EINVAL, "lmhead_topk_sample: H=%d must be a positive multiple of %d", H, PK_KC);
  if (packed_tiles_m(M) > PK_GRID)
    return fail(GRAFT_EINVAL, "lmhead_topk_sample: M=%d exceeds the packed path's %d rows", M, PK_GRID * BM);
  if (static_cast<size_t>(M) * H * 2 > 0xFFFFFFFFull)
    return fail(GRAFT_EINVAL, "lmhead_topk_sample: hidden of %d x %d exceeds 4 GiB (32-bit DMA offsets)", M, H);
  if (M == 0) return GRAFT_OK;
  if (!hidden || !w_packed || !gumbel || !topk_id || !sample_id)
    return fail(GRAFT_EINVAL, "lmhead_topk_sample: NULL array");
  if (!graft::aligned16(hidden) || !graft::aligned16(w_packed) || !graft::aligned16(gumbel))
    return fail(GRAFT_EINVAL, "lmhead_topk_sample: hidden, w_packed and gumbel must be 16-byte aligned");
  const size_t need = packed_sample_ws_bytes(M, k);
  if (ws_bytes < need || !ws) return fail(GRAFT_EINVAL, "lmhead_topk_sample: workspace %zu bytes < %zu", ws_bytes, need);
  graft::clear_error();
  hipStream_t s = graft::as_stream(stream);
  const int tiles_m = packed_tiles_m(M);
  const int tiles_v = (V + PK_BV - 1) / PK_BV;
  const int S = pk_map(0, tiles_m).streams;
  uint64_t *pk = static_cast<uint64_t *>(ws);
  uint64_t *ps = pk + static_cast<size_t>(M) * S * k;
  const float inv_temp = 1.0f / temperature;
  const unsigned char *wpk = reinterpret_cast<const unsigned char *>(w_packed);
  if (k <= 8)
    hipLaunchKernelGGL((lmhead_packed_kernel<true, 8, PK_WAVES, true>), dim3(PK_GRID), dim3(PK_WAVES * 64), 0, s, M, H, V,
                       k, hidden, wpk, nullptr, pk, tiles_m, tiles_v, inv_temp, gumbel, ps);
  else
    hipLaunchKernelGGL((lmhead_packed_kernel<true, 16, PK_WAVES, true>), dim3(PK_GRID), dim3(PK_WAVES * 64), 0, s, M, H,
                       V, k, hidden, wpk, nullptr, pk, tiles_m, tiles_v, inv_temp, gumbel, ps);
  int rc = graft::check_launch("lmhead (packed, fused top-k + sample)");
  if (rc != GRAFT_OK) return rc;
  rc = graft::launch_topk_merge(M, S, k, pk, topk_id, topk_val, s);
  if (rc != GRAFT_OK) return rc;
  return graft::launch_topk_merge(M, S, 1, ps, sample_id, nullptr, s);
}

// ------------------------------------------------- no-allocation variant
// graft_lmhead_topk's fused packed mode with its workspace (the per-(row,
// workgroup) candidate lists the merge reads) in a file-scope device array
// instead of a caller buffer, for callers that cannot allocate.  Each GPU
// holds its own copy of the array; its address is taken once per device with
// that device current and kept.  Every list the merge reads is written by the
// same call, so nothing needs clearing; calls that overlap on one GPU share
// the array and race.
namespace {
constexpr size_t kNoAllocScratchBytes = GRAFT_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The device address of this device's scratch array (nullptr + message on failure).
void *scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" size_t graft_lmhead_topk_noalloc_bytes(int M, int k) {
  if (M <= 0 || k < 1 || k > GRAFT_MAX_K || packed_tiles_m(M) > PK_GRID) return 0;
  return packed_fused_ws_bytes(M, k);
}

extern "C" int graft_lmhead_topk_noalloc(int M, int H, int V, int k, const graft_bf16 *hidden,
                                         const graft_bf16 *w_packed, int32_t *topk_id, float *topk_val,
                                         graft_stream stream) {
  using graft::fail;
  if (M < 0 || V <= 0 || V > GRAFT_MAX_V || k < 1 || k > GRAFT_MAX_K || k > V)
    return fail(GRAFT_EINVAL, "lmhead_topk_noalloc: M=%d V=%d k=%d", M, V, k);
  if (!hidden || !w_packed || !topk_id) return fail(GRAFT_EINVAL, "lmhead_topk_noalloc: NULL array");
  if (packed_tiles_m(M) > PK_GRID)
    return fail(GRAFT_EINVAL, "lmhead_topk_noalloc: M=%d exceeds the packed path's %d rows", M, PK_GRID * BM);
  const size_t need = packed_fused_ws_bytes(M, k);
  if (need > kNoAllocScratchBytes)
    return fail(GRAFT_EINVAL, "lmhead_topk_noalloc: M=%d, k=%d need %zu bytes of scratch, above the %zu built in", M,
                k, need, kNoAllocScratchBytes);
  if (M == 0) return GRAFT_OK;
  void *ws = scratch_on_current_device();
  if (!ws) return fail(GRAFT_EHIP, "lmhead_topk_noalloc: no scratch address on the current device");
  return graft_lmhead_topk(M, H, V, k, hidden, w_packed, GRAFT_W_PACKED, nullptr, topk_id, topk_val, ws,
                           kNoAllocScratchBytes, stream);
}
