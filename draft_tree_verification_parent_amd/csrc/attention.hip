// Tree-masked grouped-query attention of the flattened tree against the KV
// cache (Graft page, arXiv:2605.20104 write-up, section 2, third step: one
// parallel verification of the flattened tree with the rebuilt mask;
// TreeGraft page, section 3 and section 7 item 1: tree attention).
//
// Query row (node i, head h) sees cache slots 0..ctx-1 and tree slot ctx+j
// iff bit j of mask[i].  All N tree nodes times the G = Hq/Hkv heads of one
// KV head share every K/V tile, so a workgroup takes a key range of one
// (request, KV head) for up to 384 of its query rows at once (all N*G of
// them up to N*G = 384, the case of a 64-node tree with G <= 6): each K/V
// chunk is read from HBM once per row group, and both products run on MFMA:
//   S^T = K . Q^T   (A = K tile from LDS, B = Q fragments kept in registers)
//   O^T = V^T . P^T (A = V^T fragments from LDS, B = P straight from the S^T
//                    accumulators, re-packed to bf16)
// Computing the transposes puts one query row per lane column in both
// accumulators, so the online-softmax statistics of a row live in one lane
// group and rescaling O needs no cross-lane traffic.  A V_MFMA_F32_16X16X32
// lane holds keys {4g..4g+3} and {16+4g..16+4g+3} of its row after the S^T
// step; the P^T operand uses exactly that key set, and so does the V^T
// fragment, so no shuffle is needed between the two products.
//
// Staging: K and V chunks of 64 keys are copied HBM -> LDS in their cache
// layout by LDS DMA (global_load_lds_dwordx4: no registers, no VALU) into a
// 4-stage ring, with each key row's 16-byte pieces XOR-swizzled so that the
// fragment reads below are free of bank conflicts.  K fragments are plain
// 16-byte LDS reads; V^T fragments come from ds_read_b64_tr_b16, whose
// 16-lane transpose turns 4 keys x 16 head-dim columns of V into each lane
// holding 4 keys of one column (two reads per fragment).
//
// Work is dealt stream-K: the 64-key chunks of all (request, KV head, row
// group) units form one sequence cut into equal ranges, one per workgroup,
// so that ragged context lengths do not leave CUs idle behind the longest
// request and a few KV heads still fill 256 CUs.  A unit whose chunks one
// workgroup covers is normalised and written as bf16 there; a unit cut by a
// range boundary leaves unnormalised O, the running max and the exp-sum per
// piece, which a merge kernel combines with the usual log-sum-exp weights.
#include <cmath>
#include <type_traits>

#include "common.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int KCH = 64;      // keys per staged chunk (four 16-key MFMA blocks)
constexpr int NS = 4;        // LDS ring stages (128 KB at d = 128: one workgroup per CU)
// Fewest chunks a workgroup is given: below about eight a workgroup's fixed
// costs (first loads, the partial it writes and the merge reads back)
// dominate (one request at 4K context, 8 KV heads: 22.9 us with about 4 chunks
// per workgroup, 22.8 us with 8 at half the partial traffic, 30.5 us with 16).
constexpr int MIN_CHUNKS = 8;
constexpr int kMaxWorkgroups = 256;  // one per CU
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ inline bf16x8 zero8() { return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u}); }
__device__ inline u32x4 load16(const graft_bf16 *p) { return *reinterpret_cast<const u32x4 *>(p); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;

// Geometry of one ring stage for head dim D: the K chunk then the V chunk,
// each 64 key rows of D bf16 in cache order.  Row r keeps 16-byte piece p at
// slot p ^ swz(r); K and V use different swizzles because they are read with
// different lane patterns (16 consecutive rows of one piece for K; 8 rows x
// 2 pieces per half-wave for the V transpose reads).
template <int D>
struct Tile {
  static constexpr int ROW = D * 2;            // bytes per key row
  static constexpr int RPB = 256 / ROW;        // rows per 256-byte LDS bank line
  static constexpr int KB = KCH * ROW;         // bytes of the K (or V) chunk
  static constexpr int SB = 2 * KB;            // bytes per ring stage
  static constexpr int DI = KB / 1024 / kWaves;  // DMA instructions per wave for K (and for V)
  static_assert(DI >= 1, "each wave copies at least one KiB of K and of V");
  __device__ static int swz_k(int r) { return (r / RPB) & (D / 8 - 1); }
  __device__ static int swz_v(int r) { return 2 * ((r / RPB) & (D / 16 - 1)); }
};

// 16-byte LDS DMA (lane l's bytes from sbase + voff land at LDS byte lds +
// 16 l), issued through asm so that the compiler does not serialise the ring
// with conservative waits; completion is tracked by hand with vmcnt.
__device__ inline void lds_dma16(unsigned lds, const void *sbase, unsigned voff) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(sbase)
               : "memory", "m0");
}
// Max / sum over the 4 lanes l16, l16+16, l16+32, l16+48 (the lane groups
// that hold one query row), with the gfx950 row-swap permutes: VALU only,
// no LDS traffic.
__device__ inline float group4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float group4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// A wave-uniform pointer the compiler may keep in registers loaded per lane
// (a vector load of kv_off), moved to scalar registers for the DMA base.
__device__ inline const unsigned char *uniform_ptr(const unsigned char *p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const unsigned char *>((static_cast<uint64_t>(hi) << 32) | lo);
}
// Wait until at most N of this wave's DMAs are outstanding and its LDS
// accesses have completed, then meet the other waves.
template <int N>
__device__ inline void ring_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

struct Params {
  int B, Hq, Hkv, G;
  float scale_log2;
  const graft_bf16 *q;
  const graft_bf16 *kc;
  const graft_bf16 *vc;
  const int64_t *kv_off;
  int64_t head_stride;
  const int32_t *ctx_len;
  int max_ctx;
  const int32_t *n;
  int max_n;
  const int32_t *row_off;
  const uint64_t *mask;
  int nwg, rows_per_wg, row_groups, slot_rows;
  graft_bf16 *out;
  float *lse;
  float *ws_o;     // [2 nwg][slot_rows][D] partial O (unnormalised)
  float *ws_ml;    // [2 nwg][slot_rows][2] partial (running max, exp-sum)
  int32_t *ws_pre; // [B + 1] chunk offsets of the requests, written by workgroup 0
  int32_t *err;
};

// Per-request scalars read through the constant address space: scalar
// loads, which the compiler does not count against the vector-memory
// counter that tracks the DMA ring (the arrays are not written here).
template <typename T>
__device__ inline T ld_scalar(const T *p) {
  return *(const __attribute__((address_space(4))) T *)p;
}

// One request's scalars.
struct Request {
  int ctx, n, r_off;
  int64_t kv_off;
};

// False when the request's lengths exceed the bounds the launch was sized
// for or its row capacity, or its K/V offset is not a multiple of 8
// elements (K/V rows are copied 16 bytes at a time from kv_off[b] on);
// report: raise the matching error flag.
__device__ inline bool request_valid(const Params &P, const Request &q, int r_end, bool report) {
  const bool ok = (q.ctx >= 0) & (q.ctx <= P.max_ctx) & (q.n >= 1) & (q.n <= P.max_n) &
                  (q.n <= GRAFT_MAX_NODES) & (q.n <= r_end - q.r_off);
  const bool aligned = (q.kv_off & 7) == 0;
  if (report) {
    if (!ok) graft::raise_flag(P.err, GRAFT_ERR_CAPACITY);
    if (!aligned) graft::raise_flag(P.err, GRAFT_ERR_ALIGN);
  }
  return ok & aligned;
}

// Loads the scalars of request b (b wave-uniform) and validates them
// (report: raise the error flags).  All five loads are issued together:
// with short-circuit tests between them, each would wait for the one
// before, a chain of round trips ahead of the first K/V copy.
__device__ inline bool request_ok(const Params &P, int b, Request &q, bool report = false) {
  q.kv_off = ld_scalar(P.kv_off + b);
  q.ctx = ld_scalar(P.ctx_len + b);
  q.n = ld_scalar(P.n + b);
  q.r_off = ld_scalar(P.row_off + b);
  const int r_end = ld_scalar(P.row_off + b + 1);
  // one use of all five, and nothing scheduled across it: the loads are all
  // issued before the single wait for them
  asm volatile("" ::"s"(q.kv_off), "s"(q.ctx), "s"(q.n), "s"(q.r_off), "s"(r_end));
  __builtin_amdgcn_sched_barrier(0);
  return request_valid(P, q, r_end, report);
}

// One segment: keys [k_begin, k_end) of unit (request b, KV head h, row
// group rg) for all of the unit's query rows.  full: the segment is the
// unit's whole key range, and the normalised bf16 output (and LSE) is
// written; otherwise the unnormalised partial (O, running max, exp-sum) goes
// to workspace slot `slot`.  Every thread of the workgroup calls it.
template <int D, int RBW>
__device__ __forceinline__ void attend_segment(const Params &P, unsigned char *sm, int b, int h, int rg,
                                               const Request &q, int k_begin, int k_end, bool full, int slot) {
  using TL = Tile<D>;
  constexpr int DS = D / 32;  // MFMA k-steps over the head dim
  constexpr int DB = D / 16;  // 16-wide output blocks over the head dim
  constexpr int DI = TL::DI;

  const int ctx = q.ctx, n = q.n;
  const int rows_total = n * P.G;
  const int row_lo = rg * P.rows_per_wg;
  if (row_lo >= rows_total) return;
  const int nch = (k_end - k_begin + KCH - 1) / KCH;

  // the lane-dependent offsets below are recomputed per segment rather than
  // hoisted out of the segment loop, where they would stay live across it
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g = lane >> 4;
  const int r_off = q.r_off;

  // ---- LDS DMA ring.  Lane l of this wave's i-th K (V) instruction copies
  // piece (slot ^ swz(row)) of key row `row` of the chunk into slot `slot`.
  // Slots past k_end re-read the last valid slot (in bounds; their scores
  // are masked and their P is 0).
  const unsigned sbase = static_cast<unsigned>(reinterpret_cast<size_t>((lds_u8 *)sm));
  const size_t kv_base = static_cast<size_t>(q.kv_off) + static_cast<size_t>(h) * P.head_stride;
  const unsigned char *kbase = uniform_ptr(reinterpret_cast<const unsigned char *>(P.kc + kv_base));
  const unsigned char *vbase = uniform_ptr(reinterpret_cast<const unsigned char *>(P.vc + kv_base));
  int drow[DI];
  unsigned kpc[DI], vpc[DI];
#pragma unroll
  for (int i = 0; i < DI; ++i) {
    const int byte = (wave * DI + i) * 1024 + lane * 16;
    const int r = byte / TL::ROW;
    const int slot = (byte - r * TL::ROW) / 16;
    drow[i] = r;
    kpc[i] = ((slot ^ TL::swz_k(r)) * 16);
    vpc[i] = ((slot ^ TL::swz_v(r)) * 16);
  }
  auto issue = [&](int c) {
    const int c0 = k_begin + c * KCH;
    const unsigned kl = sbase + (c % NS) * TL::SB + wave * DI * 1024;
#pragma unroll
    for (int i = 0; i < DI; ++i) {
      const unsigned srow = static_cast<unsigned>(min(c0 + drow[i], k_end - 1)) * TL::ROW;
      lds_dma16(kl + i * 1024, kbase, srow + kpc[i]);
      lds_dma16(kl + TL::KB + i * 1024, vbase, srow + vpc[i]);
    }
  };

  // ---- ring prologue first: chunks 0 .. NS-2 go in flight before anything
  // else is loaded
#pragma unroll
  for (int c = 0; c < NS - 1; ++c)
    if (c < nch) issue(c);

  // ---- this lane's query rows: Q fragments and tree-mask words (their
  // latency overlaps the first chunks')
  bf16x8 qf[RBW][DS];
  uint64_t mrow[RBW];
  bool rvalid[RBW];
  bool active[RBW];
#pragma unroll
  for (int j = 0; j < RBW; ++j) {
    // row blocks are dealt round-robin (block j * 8 + wave), so the two waves
    // of each SIMD carry at most one block more than any other pair
    const int rb0 = row_lo + (j * kWaves + wave) * 16;
    // wave-uniform; readfirstlane lets the compiler branch on a scalar
    // instead of masking every MFMA below
    active[j] = __builtin_amdgcn_readfirstlane(rb0 < rows_total ? 1 : 0) != 0;
    const int r = rb0 + l16;
    rvalid[j] = r < rows_total;
    const int node = (rvalid[j] ? r : 0) / P.G;
    const int hq = h * P.G + ((rvalid[j] ? r : 0) - node * P.G);
    mrow[j] = rvalid[j] ? P.mask[r_off + node] : 0ull;
    const graft_bf16 *qp = P.q + (static_cast<size_t>(r_off + node) * P.Hq + hq) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < DS; ++s) qf[j][s] = rvalid[j] ? __builtin_bit_cast(bf16x8, load16(qp + s * 32)) : zero8();
  }

  // Retire the Q and mask loads here.  The compiler does not see the DMAs
  // (they are asm), so its own wait for these loads, placed at their first
  // use inside the ring loop, would be a vmcnt(0) run on every chunk: each
  // chunk would wait for every DMA in flight, the ring would never overlap
  // compute.  Used once here, they cost one wait that also covers the
  // prologue's chunks, which the first chunk needs anyway.
#pragma unroll
  for (int j = 0; j < RBW; ++j) {
    asm volatile("" ::"v"(mrow[j]));
#pragma unroll
    for (int s = 0; s < DS; ++s) asm volatile("" ::"v"(qf[j][s]));
  }

  f32x4 oacc[RBW][DB];
  float m_run[RBW], l_run[RBW];
#pragma unroll
  for (int j = 0; j < RBW; ++j) {
    m_run[j] = -INFINITY;
    l_run[j] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[j][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // per-lane fragment offsets (the swizzles depend only on the lane)
  const int swk = TL::swz_k(l16);                  // K rows 32t + 16kb + l16
  const int vr = 4 * g + (l16 >> 2);               // V rows 32t + vr (+16)
  const int swv = TL::swz_v(vr);
  const int vcol = 4 * (l16 & 3);                  // first head-dim column within the 16-block
  const int kfrag = l16 * TL::ROW;
  const int vfrag = vr * TL::ROW + 8 * ((vcol >> 2) & 1);

  // A chunk's work in three phases: S^T for its 64 keys (MFMA), one
  // online-softmax update per row block (VALU), then O^T += V^T . P^T over
  // its two 32-key halves (MFMA).  NA, the number of active row blocks
  // (always the first NA), is a compile-time constant so the MFMAs carry no
  // branches and the fragment reads can be issued ahead of them.
  auto s_phase = [&](auto na_tag, int c, f32x4(&sacc)[RBW][4]) {
    constexpr int NA = decltype(na_tag)::value;
    const lds_u8 *ks = (const lds_u8 *)sm + (c % NS) * TL::SB;
    // S^T blocks: sacc[j][kb][i] = S[row l16][key c0 + kb*16 + 4g + i]
#pragma unroll
    for (int j = 0; j < NA; ++j)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) sacc[j][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (NA <= 2) {
      // registers to spare: all 4 x DS K fragments are read first, in the
      // order the MFMAs consume them, and the MFMAs run k-step by k-step
      // over the four key blocks, so consecutive MFMAs never depend on each
      // other and each waits only for its own fragment
      bf16x8 kf[DS][4];
#pragma unroll
      for (int s = 0; s < DS; ++s)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          kf[s][kb] = *(const __attribute__((address_space(3))) bf16x8 *)(ks + 16 * kb * TL::ROW + kfrag +
                                                                          (((4 * s + g) ^ swk) * 16));
      __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMAs
#pragma unroll
      for (int s = 0; s < DS; ++s)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int j = 0; j < NA; ++j)
            sacc[j][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s][kb], qf[j][s], sacc[j][kb], 0, 0, 0);
    } else {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int s = 0; s < DS; ++s) {
          const bf16x8 a = *(const __attribute__((address_space(3))) bf16x8 *)(
              ks + 16 * kb * TL::ROW + kfrag + (((4 * s + g) ^ swk) * 16));
#pragma unroll
          for (int j = 0; j < NA; ++j)
            sacc[j][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[j][s], sacc[j][kb], 0, 0, 0);
        }
      }
    }
  };
  auto x_phase = [&](auto na_tag, int c, const f32x4(&sacc)[RBW][4], bf16x8(&pb)[RBW][2]) {
    constexpr int NA = decltype(na_tag)::value;
    const int c0 = k_begin + c * KCH;
    // online softmax (base 2).  A chunk that lies entirely inside the
    // context needs no mask (uniform test).
    const bool unmasked = c0 + KCH <= ctx && c0 + KCH <= k_end;
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      // raw scores; the scale is folded into the exp2 argument below
      float x[16];
      if (unmasked) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[kb * 4 + i] = sacc[j][kb][i];
      } else {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = c0 + kb * 16 + 4 * g + i;
            const bool tree_vis = ((mrow[j] >> ((key - ctx) & 63)) & 1ull) != 0;
            const bool vis = (key < k_end) & ((key < ctx) | tree_vis);  // no short-circuit branches
            x[kb * 4 + i] = vis ? sacc[j][kb][i] : -INFINITY;
          }
      }
      float cmax = x[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) cmax = fmaxf(cmax, x[e]);
      cmax = group4_max(cmax) * P.scale_log2;  // scale > 0: max commutes with it
      // Lazy rescaling: the running max m only moves when some row of the
      // wave sees a score more than 8 (log2 units) above it, so p stays
      // <= 2^8 and O, l keep sharing the same m (the final O / l is
      // unchanged); most chunks then skip the O rescale entirely.
      const bool grow = cmax > m_run[j] + 8.f;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {  // wave-uniform
        // rows that do not grow keep alpha = 1 (also when m is still -inf)
        const float alpha = grow ? __builtin_amdgcn_exp2f(m_run[j] - cmax) : 1.f;  // 0 from -inf
        l_run[j] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[j][db] *= alpha;
        m_run[j] = grow ? cmax : m_run[j];
      }
      // rows with nothing visible yet keep m = -inf: shift by 0 (p = 0)
      const float m_use = m_run[j] == -INFINITY ? 0.f : m_run[j];
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        x[e] = __builtin_amdgcn_exp2f(fmaf(x[e], P.scale_log2, -m_use));
        psum += x[e];
      }
      l_run[j] += psum;
      // half t holds keys {32t + 4g + i} (block 2t) and {32t + 16 + 4g + i}
      // (block 2t + 1)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[j][t][e] = static_cast<__bf16>(x[8 * t + e]);
    }
  };
  auto o_phase = [&](auto na_tag, int c, const bf16x8(&pb)[RBW][2]) {
    constexpr int NA = decltype(na_tag)::value;
    const lds_u8 *vs = (const lds_u8 *)sm + (c % NS) * TL::SB + TL::KB;
    // O^T += V^T . P^T: lane (d = db*16 + l16, g) needs keys {4g..4g+3}
    // and {16+4g..16+4g+3} of the half for head-dim column d; the 16-lane
    // transpose read delivers them when lane a of the group points at key
    // row 4g + a/4, columns db*16 + 4(a%4) .. +3.
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int piece = 2 * db + ((vcol >> 3) & 1);
        const lds_u8 *va = vs + 32 * t * TL::ROW + vfrag + ((piece ^ swv) * 16);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)va);
        const s16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(va + 16 * TL::ROW));
        const u32x2 lw = __builtin_bit_cast(u32x2, lo);
        const u32x2 hw = __builtin_bit_cast(u32x2, hi);
        const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{lw[0], lw[1], hw[0], hw[1]});
#pragma unroll
        for (int j = 0; j < NA; ++j)
          oacc[j][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[j][t], oacc[j][db], 0, 0, 0);
      }
    }
  };

  // ---- ring: chunks c+1 .. c+NS-2 stay in flight while chunk c is computed.
  // A wave without active row blocks still issues its share of every
  // chunk's DMAs and meets the others at each barrier.  (Running the two
  // waves of each SIMD half a chunk apart, one in its softmax while the
  // other runs its products, measured no faster.)
  constexpr int PER = 2 * DI;  // DMAs per wave per chunk
  auto run = [&](auto na_tag) {
    constexpr int NA = decltype(na_tag)::value;
    for (int c = 0; c < nch; ++c) {
      static_assert(NS - 2 <= 2, "the waits below cover at most two younger chunks");
      const int younger = min(nch - 1 - c, NS - 2);  // chunks issued after c
      if (younger >= 2) ring_barrier<2 * PER>();
      else if (younger == 1) ring_barrier<PER>();
      else ring_barrier<0>();
      if (c + NS - 1 < nch) issue(c + NS - 1);  // into the stage chunk c - 1 used
      if constexpr (NA > 0) {
        f32x4 sacc[RBW][4];  // S^T of the chunk
        bf16x8 pb[RBW][2];   // P^T operand of each 32-key half
        s_phase(na_tag, c, sacc);
        x_phase(na_tag, c, sacc, pb);
        o_phase(na_tag, c, pb);
      }
    }
  };
  int nact = 0;  // active row blocks are the first nact (wave-uniform)
#pragma unroll
  for (int j = 0; j < RBW; ++j) nact += active[j] ? 1 : 0;
  if (nact == 0) run(std::integral_constant<int, 0>{});
  else if (RBW == 1 || nact == 1) run(std::integral_constant<int, 1>{});
  else if (RBW == 2 || nact == 2) run(std::integral_constant<int, (RBW >= 2 ? 2 : 1)>{});
  else run(std::integral_constant<int, (RBW >= 3 ? 3 : 1)>{});

  // ---- epilogue: oacc[j][db][i] = O[row l16][d = db*16 + 4g + i]
#pragma unroll
  for (int j = 0; j < RBW; ++j) {
    if (!active[j]) continue;
    const float l_tot = group4_sum(l_run[j]);
    if (!rvalid[j]) continue;
    const int r = row_lo + (j * kWaves + wave) * 16 + l16;
    if (full) {
      const int node = r / P.G;
      const int hq = h * P.G + (r - node * P.G);
      const size_t orow = static_cast<size_t>(r_off + node) * P.Hq + hq;
      const float inv = 1.f / l_tot;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        bf16x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = static_cast<__bf16>(oacc[j][db][i] * inv);
        *reinterpret_cast<bf16x4 *>(P.out + orow * D + db * 16 + 4 * g) = o;
      }
      if (P.lse && g == 0) P.lse[orow] = (m_run[j] + log2f(l_tot)) * kLn2;
    } else {
      const size_t srow = static_cast<size_t>(slot) * P.slot_rows + (r - row_lo);
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<f32x4 *>(P.ws_o + srow * D + db * 16 + 4 * g) = oacc[j][db];
      if (g == 0) {
        P.ws_ml[srow * 2] = m_run[j];
        P.ws_ml[srow * 2 + 1] = l_tot;
      }
    }
  }
}

// A unit is one (KV head, row group) of a request that has rows in that
// group: Hkv * ceil(n G / rows_per_wg) units, taken KV head by KV head, each
// of ceil((ctx + n) / 64) chunks (a request skipped as invalid has none).
__device__ inline int unit_chunks(const Request &q, bool ok) { return ok ? (q.ctx + q.n + KCH - 1) / KCH : 0; }
__device__ inline int live_groups(const Params &P, const Request &q) {
  return (q.n * P.G + P.rows_per_wg - 1) / P.rows_per_wg;
}

// The requests' chunk offsets (a workgroup scan over their lengths, into
// s_pre; workgroup 0 also stores them for the merge and raises the
// requests' error flags), and where workgroup w's range starts: out = {T,
// the request b holding chunk s_w, s_w - s_pre[b]}.  Thread t owns requests
// t * PT .. t * PT + PT - 1; a wave scan of the owners' sums and a scan of
// the wave totals give each owner its starting offset.  Loops here are
// fully unrolled: a loop ahead of the segment loop changed how the
// segments' registers were allocated and pushed the 3-row-block variant
// into spills.
__device__ inline void stream_start(const Params &P, int *s_pre, int *s_wsum, int *out) {
  constexpr int PT = (GRAFT_ATTN_MAX_BATCH + kThreads - 1) / kThreads;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int mine = 0;
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int b = tid * PT + i;
    if (b < P.B) {
      Request q;
      q.kv_off = P.kv_off[b];
      q.ctx = P.ctx_len[b];
      q.n = P.n[b];
      q.r_off = P.row_off[b];
      const bool ok = request_valid(P, q, P.row_off[b + 1], blockIdx.x == 0);
      const int cnt = unit_chunks(q, ok) * P.Hkv * live_groups(P, q);
      s_pre[b] = cnt;
      mine += cnt;
    }
  }
  int incl = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int run = incl - mine;
#pragma unroll
  for (int w2 = 0; w2 < kWaves; ++w2) run += w2 < wave ? s_wsum[w2] : 0;
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int b = tid * PT + i;
    if (b < P.B) {
      const int cnt = s_pre[b];
      s_pre[b] = run;
      run += cnt;
    }
  }
  if (tid == kThreads - 1) s_pre[P.B] = run;  // run: the total T
  __syncthreads();
  const int T = s_pre[P.B];
  if (blockIdx.x == 0) {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int b = tid * PT + i;
      if (b < P.B) P.ws_pre[b] = s_pre[b];
    }
    if (tid == 0) P.ws_pre[P.B] = T;  // (b = B is past the owners' range when B = GRAFT_ATTN_MAX_BATCH)
  }
  const int s_w = static_cast<int>(static_cast<long long>(blockIdx.x) * T / P.nwg);
  // the request holding chunk s_w: s_pre[b] <= s_w < s_pre[b + 1] (one
  // request, when s_w < T)
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int b = tid * PT + i;
    if (b < P.B && s_pre[b] <= s_w && s_w < s_pre[b + 1]) {
      out[1] = b;
      out[2] = s_w - s_pre[b];
    }
  }
  if (tid == 0) out[0] = T;
}

// Stream-K over the chunk sequence: the units (request, KV head, row group)
// in order, each ceil((ctx + n) / 64) chunks long.  Workgroup w of nwg takes
// chunks [w T / nwg, (w + 1) T / nwg) of the T in all, so every workgroup
// gets the same number of chunks whatever the requests' lengths.  A unit
// that one workgroup covers whole is finished there; a unit cut by a range
// boundary leaves partials (at most two per workgroup, its first and its
// last segment: slots 2w and 2w + 1) that tree_attn_merge_kernel combines.
// The per-request chunk offsets come from a workgroup scan over the
// requests' lengths, kept in the (not yet used) ring LDS; workgroup 0 also
// stores them for the merge and raises the requests' error flags.
template <int D, int RBW>
__global__ __launch_bounds__(kThreads, 2) void tree_attn_kernel(Params P) {
  using TL = Tile<D>;
  __shared__ __attribute__((aligned(1024))) unsigned char sm[NS * TL::SB];
  __shared__ int s_wsum[kWaves];
  static_assert(NS * TL::SB >= 4 * (GRAFT_ATTN_MAX_BATCH + 1), "request offsets fit the ring");
  int *s_pre = reinterpret_cast<int *>(sm);
  const int tid = threadIdx.x;

  // where this workgroup's range starts: chunk s_w, in request b at offset
  // o.  One request needs no scan.
  __shared__ int s_start[3];
  int T;
  if (P.B == 1) {
    Request q;
    const bool ok = request_ok(P, 0, q, blockIdx.x == 0 && tid == 0);
    T = unit_chunks(q, ok) * P.Hkv * live_groups(P, q);
    if (blockIdx.x == 0 && tid == 0) {
      P.ws_pre[0] = 0;
      P.ws_pre[1] = T;
    }
  } else {
    stream_start(P, s_pre, s_wsum, s_start);
    __syncthreads();
    T = __builtin_amdgcn_readfirstlane(s_start[0]);
  }
  const int w = blockIdx.x;
  const int s_w = static_cast<int>(static_cast<long long>(w) * T / P.nwg);
  const int e_w = static_cast<int>(static_cast<long long>(w + 1) * T / P.nwg);
  if (s_w >= e_w) return;
  int b = 0, o = s_w;
  if (P.B != 1) {
    b = __builtin_amdgcn_readfirstlane(s_start[1]);
    o = __builtin_amdgcn_readfirstlane(s_start[2]);
    __syncthreads();  // every wave has read s_pre before the ring overwrites it
  }

  // The walk's next state (request, unit, position) waits in LDS while a
  // segment runs, so that no register is held across the segment for it
  // (the request's scalars are loaded again per segment: scalar-cache
  // hits).  Two copies, by segment parity: thread 0 writes the next
  // segment's copy while slower waves may still be reading this one (the
  // barriers inside a segment then order the copy they read against its
  // next rewrite).
  __shared__ int s_walk[2][4];
  int ui, c, gpos = s_w, par = 0;
  {
    Request q;
    const int nch = unit_chunks(q, request_ok(P, b, q));  // the request holds chunk s_w
    ui = o / nch;
    c = o - ui * nch;
  }
  for (;;) {
    Request q;
    const int nch = unit_chunks(q, request_ok(P, b, q));  // > 0: the request holds chunk gpos
    const int rgl = live_groups(P, q);
    const int len = min(e_w - gpos, nch - c);
    const int h = ui / rgl;
    const int rg = ui - h * rgl;
    const int L = q.ctx + q.n;
    volatile int *walk = s_walk[par];
    if (tid == 0) {
      // the next unit: the next (KV head, row group), else the next request
      // with chunks (the walk stops before passing the last)
      int nb = b, nu = ui + 1;
      if (nu == P.Hkv * rgl) {
        nu = 0;
        ++nb;
      }
      walk[0] = nb;
      walk[1] = nu;
      walk[2] = gpos + len;
    }
    attend_segment<D, RBW>(P, sm, b, h, rg, q, c * KCH, min(L, (c + len) * KCH), c == 0 && len == nch,
                           2 * w + (gpos == s_w ? 0 : 1));
    __syncthreads();  // every wave is done with the ring before it refills; walk[] is written
    gpos = __builtin_amdgcn_readfirstlane(walk[2]);
    if (gpos >= e_w) break;
    b = __builtin_amdgcn_readfirstlane(walk[0]);
    ui = __builtin_amdgcn_readfirstlane(walk[1]);
    c = 0;
    par ^= 1;
    if (ui == 0)  // skip requests without chunks (invalid ones)
      while (unit_chunks(q, request_ok(P, b, q)) == 0) ++b;
  }
  // the ring's last DMAs were waited for inside the segment
}

// Combines the partials of the units that no single workgroup covered, one
// query row of one KV head per D/4 lanes, each lane owning 4 head-dim
// columns: the workgroups over the unit are the non-empty ones from the
// one holding its first chunk to the one holding its last; the first uses
// its second slot when its range began before the unit, every other one its
// first slot.  One pass with a running
// maximum, the slot loads unrolled so that their latencies overlap.
template <int D>
__global__ __launch_bounds__(256) void tree_attn_merge_kernel(Params P) {
  constexpr int TPR = D / 4;      // threads per row
  constexpr int RPB = 256 / TPR;  // rows per block
  const int b = blockIdx.z;
  const int h = blockIdx.y;
  const int r = blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = (threadIdx.x % TPR) * 4;
  Request q;
  if (!request_ok(P, b, q)) return;
  if (r >= q.n * P.G) return;
  const int nch = unit_chunks(q, true);
  const int rg = r / P.rows_per_wg;
  // the chunk count and the unit's first chunk (one request: no loads)
  const int rgl = live_groups(P, q);
  const int T = P.B == 1 ? P.Hkv * rgl * nch : P.ws_pre[P.B];
  const int A = (P.B == 1 ? 0 : P.ws_pre[b]) + (h * rgl + rg) * nch;
  // The offsets come from the attention kernel of the same call; whatever
  // they hold, every slot read below stays inside the 2 nwg slots.
  if (T <= 0 || A < 0 || A > T - nch) return;
  // workgroup holding chunk x: the last w with floor(w T / nwg) <= x
  auto owner = [&](int x) { return static_cast<int>((static_cast<long long>(x + 1) * P.nwg + T - 1) / T) - 1; };
  const int w0 = max(0, owner(A)), w1 = min(P.nwg - 1, owner(A + nch - 1));
  if (w0 >= w1) return;  // finished by that workgroup
  const bool w0_late = static_cast<long long>(w0) * T / P.nwg < A;
  const bool sparse = T < P.nwg;  // else every workgroup's range holds a chunk
  const int rr = r - rg * P.rows_per_wg;
  float M = -INFINITY, wsum = 0.f;
  f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int U = 8;
  for (int w = w0; w <= w1; w += U) {
    float ms[U], ls[U];
    f32x4 os[U];
    bool use[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int wu = min(w + u, w1);
      const int slot = 2 * wu + ((wu == w0 && w0_late) ? 1 : 0);
      const size_t srow = static_cast<size_t>(slot) * P.slot_rows + rr;
      // with fewer chunks than workgroups some ranges are empty: those
      // workgroups wrote nothing
      use[u] = w + u <= w1 &&
               (!sparse || static_cast<long long>(wu) * T / P.nwg < static_cast<long long>(wu + 1) * T / P.nwg);
      ms[u] = P.ws_ml[srow * 2];
      ls[u] = P.ws_ml[srow * 2 + 1];
      os[u] = *reinterpret_cast<const f32x4 *>(P.ws_o + srow * D + c);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!use[u] || ms[u] == -INFINITY) continue;
      const float Mn = fmaxf(M, ms[u]);
      const float a = exp2f(M - Mn);  // 0 when M was -inf
      const float wt = exp2f(ms[u] - Mn);
      wsum = wsum * a + wt * ls[u];
      o = o * a + os[u] * wt;
      M = Mn;
    }
  }
  const int node = r / P.G;
  const int hq = h * P.G + (r - node * P.G);
  const size_t orow = static_cast<size_t>(q.r_off + node) * P.Hq + hq;
  const float inv = 1.f / wsum;
  bf16x4 ob;
#pragma unroll
  for (int i = 0; i < 4; ++i) ob[i] = static_cast<__bf16>(o[i] * inv);
  *reinterpret_cast<bf16x4 *>(P.out + orow * D + c) = ob;
  if (P.lse && c == 0) P.lse[orow] = (M + log2f(wsum)) * kLn2;
}

struct Plan {
  int rbw, row_groups, rows_per_wg, rows_cap, slot_rows, nwg;
  long long chunks;  // chunks of the largest batch the bounds allow
  size_t ws_bytes;
};

Plan make_plan(int B, int Hq, int Hkv, int d, int max_ctx, int max_n) {
  Plan p{};
  const int G = Hq / Hkv;
  const int rows = max_n * G;
  const int rb = (rows + 15) / 16;
  // Row blocks per wavefront.  With few (request, KV head) units a
  // workgroup's time is dominated by its fixed costs (first loads, partial
  // write) and lighter workgroups win (measured: 240 rows of one request at
  // 4K context, 23 us with one block per wave in two row groups against 32
  // with two blocks in one, which reads the K/V once), so one block per wave
  // is used while that makes at most two row groups and fewer than 256
  // units; otherwise the fewest row groups (each re-reads the unit's K/V),
  // up to 3 blocks per wave (4 spill at d = 128).
  const int rg1 = (rows + kWaves * 16 - 1) / (kWaves * 16);
  if (rg1 <= 2 && static_cast<long long>(B) * Hkv * rg1 < 256) p.rbw = 1;
  else p.rbw = rb <= kWaves ? 1 : rb <= 2 * kWaves ? 2 : 3;
  p.rows_per_wg = kWaves * p.rbw * 16;
  p.row_groups = (rows + p.rows_per_wg - 1) / p.rows_per_wg;
  p.rows_cap = rb * 16;
  p.slot_rows = p.rows_cap < p.rows_per_wg ? p.rows_cap : p.rows_per_wg;
  const long long L = static_cast<long long>(max_ctx) + max_n;
  p.chunks = static_cast<long long>(B) * Hkv * p.row_groups * ((L + KCH - 1) / KCH);
  // one workgroup per CU, each taking at least MIN_CHUNKS chunks.  With at
  // most half as many units as CUs the count is a multiple of the units, so
  // that when every request has the bounds' lengths (one request, or a
  // uniform batch) each range lies inside one unit and leaves one partial.
  const long long units = static_cast<long long>(B) * Hkv * p.row_groups;
  const long long nch = (L + KCH - 1) / KCH;
  long long nwg;
  if (units * 2 <= kMaxWorkgroups) {
    long long per = kMaxWorkgroups / units;
    if (per > nch / MIN_CHUNKS) per = nch / MIN_CHUNKS;
    nwg = units * (per < 1 ? 1 : per);
  } else {
    nwg = (p.chunks + MIN_CHUNKS - 1) / MIN_CHUNKS;
  }
  p.nwg = static_cast<int>(nwg < 1 ? 1 : nwg > kMaxWorkgroups ? kMaxWorkgroups : nwg);
  p.ws_bytes = static_cast<size_t>(2) * p.nwg * p.slot_rows * (d + 2) * sizeof(float) +
               (static_cast<size_t>(B) + 1) * sizeof(int32_t);
  return p;
}

bool shape_ok(int B, int Hq, int Hkv, int d, int max_ctx, int max_n) {
  return B >= 0 && Hkv > 0 && Hq > 0 && Hq % Hkv == 0 && Hq / Hkv <= 16 && (d == 64 || d == 128) &&
         max_ctx >= 0 && max_n >= 1 && max_n <= GRAFT_MAX_NODES;
}

template <int D>
void launch(const Plan &pl, const Params &P, hipStream_t s) {
  const dim3 grid(pl.nwg);
  if (pl.rbw == 1)
    hipLaunchKernelGGL((tree_attn_kernel<D, 1>), grid, dim3(kThreads), 0, s, P);
  else if (pl.rbw == 2)
    hipLaunchKernelGGL((tree_attn_kernel<D, 2>), grid, dim3(kThreads), 0, s, P);
  else
    hipLaunchKernelGGL((tree_attn_kernel<D, 3>), grid, dim3(kThreads), 0, s, P);
  if (pl.nwg > 1) {
    constexpr int RPB = 256 / (D / 4);
    dim3 mg((pl.rows_cap + RPB - 1) / RPB, P.Hkv, P.B);
    hipLaunchKernelGGL(tree_attn_merge_kernel<D>, mg, dim3(256), 0, s, P);
  }
}

}  // namespace

extern "C" size_t graft_tree_attention_workspace_bytes(int B, int Hq, int Hkv, int d, int max_ctx, int max_n) {
  if (!shape_ok(B, Hq, Hkv, d, max_ctx, max_n) || B == 0) return 0;
  return make_plan(B, Hq, Hkv, d, max_ctx, max_n).ws_bytes;
}

extern "C" int graft_tree_attention(int B, int Hq, int Hkv, int d, float scale, const graft_bf16 *q,
                                    const graft_bf16 *kcache, const graft_bf16 *vcache, const int64_t *kv_off,
                                    int64_t kv_head_stride, const int32_t *ctx_len, int max_ctx,
                                    const int32_t *n, int max_n, const int32_t *row_off, const uint64_t *mask,
                                    graft_bf16 *out, float *lse, void *ws, size_t ws_bytes, int32_t *err_flag,
                                    graft_stream stream) {
  using graft::fail;
  if (!shape_ok(B, Hq, Hkv, d, max_ctx, max_n)) {
    if (d != 64 && d != 128 && d > 0) return fail(GRAFT_EUNSUPPORTED, "tree_attention: head dim %d (built: 64, 128)", d);
    return fail(GRAFT_EINVAL, "tree_attention: B=%d Hq=%d Hkv=%d d=%d max_ctx=%d max_n=%d", B, Hq, Hkv, d, max_ctx,
                max_n);
  }
  if (B == 0) return GRAFT_OK;
  if (B > GRAFT_ATTN_MAX_BATCH)
    return fail(GRAFT_EINVAL, "tree_attention: B=%d > %d", B, GRAFT_ATTN_MAX_BATCH);
  const Plan pl = make_plan(B, Hq, Hkv, d, max_ctx, max_n);
  if (pl.chunks > INT32_MAX || Hkv > 65535)
    return fail(GRAFT_EINVAL, "tree_attention: %lld key chunks (B * Hkv * row groups * ceil((max_ctx + max_n) / 64)) "
                              "exceed 2^31 - 1", pl.chunks);
  if (!q || !kcache || !vcache || !kv_off || !ctx_len || !n || !row_off || !mask || !out)
    return fail(GRAFT_EINVAL, "tree_attention: NULL array");
  if (!graft::aligned16(q) || !graft::aligned16(kcache) || !graft::aligned16(vcache) || !graft::aligned16(out) ||
      kv_head_stride % 8 != 0)
    return fail(GRAFT_EINVAL, "tree_attention: q, kcache, vcache and out must be 16-byte aligned and "
                              "kv_head_stride a multiple of 8");
  if (kv_head_stride < static_cast<int64_t>(max_ctx + max_n) * d)
    return fail(GRAFT_EINVAL, "tree_attention: kv_head_stride %lld < (max_ctx + max_n) * d",
                static_cast<long long>(kv_head_stride));
  if (ws_bytes < pl.ws_bytes || !ws)
    return fail(GRAFT_EINVAL, "tree_attention: workspace %zu bytes < %zu", ws_bytes, pl.ws_bytes);
  if (!graft::aligned16(ws))  // partial O rows are moved 16 bytes at a time
    return fail(GRAFT_EINVAL, "tree_attention: workspace must be 16-byte aligned");
  graft::clear_error();
  Params P{};
  P.B = B;
  P.Hq = Hq;
  P.Hkv = Hkv;
  P.G = Hq / Hkv;
  P.scale_log2 = scale * kLog2e;
  P.q = q;
  P.kc = kcache;
  P.vc = vcache;
  P.kv_off = kv_off;
  P.head_stride = kv_head_stride;
  P.ctx_len = ctx_len;
  P.max_ctx = max_ctx;
  P.n = n;
  P.max_n = max_n;
  P.row_off = row_off;
  P.mask = mask;
  P.nwg = pl.nwg;
  P.rows_per_wg = pl.rows_per_wg;
  P.row_groups = pl.row_groups;
  P.slot_rows = pl.slot_rows;
  P.out = out;
  P.lse = lse;
  const size_t slots = static_cast<size_t>(2) * pl.nwg * pl.slot_rows;
  P.ws_o = static_cast<float *>(ws);
  P.ws_ml = P.ws_o + slots * d;
  P.ws_pre = reinterpret_cast<int32_t *>(P.ws_ml + slots * 2);
  P.err = err_flag;
  hipStream_t s = graft::as_stream(stream);
  if (d == 128) launch<128>(pl, P, s);
  else launch<64>(pl, P, s);
  return graft::check_launch("tree_attention");
}
