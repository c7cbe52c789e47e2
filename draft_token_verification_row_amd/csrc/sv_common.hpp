// sv_common.hpp - pieces shared by the kernels of libspecverify (gfx950):
// workspace records, the element loaders, the per-unit row statistics
// (softmax partials and argmax partials over one slice of a logit row), the
// row-statistics kernel k_stats, and host helpers.  Included once by each
// translation unit of the library; everything but the shared host state
// below has internal linkage.
#pragma once

#include <hip/hip_runtime.h>

#include <float.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "spec_verify.h"

namespace svk {
// Host state shared by every translation unit (one copy per thread).
inline thread_local void* g_ev_begin = nullptr;   // profile events (spec_verify_set_profile_events)
inline thread_local void* g_ev_end = nullptr;
inline thread_local int g_launch_plan = 0;        // 0 automatic, 1 multi-kernel, 2 single launch
}  // namespace svk

namespace {

using svk::g_ev_begin;
using svk::g_ev_end;
using svk::g_launch_plan;

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
#ifndef SV_UNROLL
#define SV_UNROLL 2
#endif
#ifndef SV_SEG_BYTES
#define SV_SEG_BYTES 32768
#endif
#ifndef SV_MALL_ORDER
#define SV_MALL_ORDER 1
#endif
constexpr int kUnroll = SV_UNROLL;       // 16-byte chunks per lane per step of a unit loop
#ifndef SV_ARGMAX_UNROLL
#define SV_ARGMAX_UNROLL 4
#endif
constexpr int kArgmaxUnroll = SV_ARGMAX_UNROLL;   // the same for argmax units (less work per chunk)
#ifndef SV_ROUND_UNROLL
#define SV_ROUND_UNROLL 4
#endif
// early-exit rounds: same per-lane chunk order (so the same partials bit for
// bit), more loads in flight for the small late rounds
constexpr int kRoundUnroll = SV_ROUND_UNROLL;
#ifndef SV_ROUND_RESID_UNROLL
#define SV_ROUND_RESID_UNROLL 1
#endif
constexpr int kRoundResidUnroll = SV_ROUND_RESID_UNROLL;   // residual pairs in the rounds
#ifndef SV_RESID_UNROLL
#define SV_RESID_UNROLL 1
#endif
constexpr int kResidUnroll = SV_RESID_UNROLL;   // k_resid: chunks per lane per row and step
constexpr int kSegBytes = SV_SEG_BYTES;  // one unit = 32 KiB of one logit row
constexpr int kSegMinElems = kSegBytes / 4;
constexpr int kRSegBytes = 8192;    // residual unit = 8 KiB of each of two rows
constexpr int kTreeSegBytes = 4096; // early-exit tree rounds: 4 KiB units (few rows per round)
constexpr int kRSegMinElems = kRSegBytes / 4;
constexpr int kBlocksPerCU = 8;      // 32 wavefronts per CU
constexpr int kPlanThreads = 1024;
constexpr int kMaxEarlyExitRounds = 4096;   // bound on max_k (two launches per round)

constexpr uint32_t kDraftBit = 1u << 30;
constexpr uint32_t kGreedyBit = 1u << 29;
constexpr uint32_t kRowMask = kGreedyBit - 1u;

enum Kind : int { KIND_NONE = 0, KIND_RESID = 1, KIND_BONUS = 2, KIND_INVALID = 3 };
enum DrawMode : int { DRAW_RESID = 0, DRAW_FROM_P = 1 };

struct Partial {      // one unit of one row
  double s;           // sum of exp2((z - m) * c) over the unit (softmax rows)
  float m;            // max logit of the unit
  int idx;            // lowest id attaining m (greedy rows)
};

struct ReqInfo {      // per request; plan fills off/k/greedy, decide the rest
  int off, k, greedy, a;
  int kind, y, trow, drow;
  float Mp, Mq;
  int pad0, pad1;
  double Sp, Sq;
};

struct __align__(16) AliveEntry {   // early exit: a request still deciding, with
  int b, off, k, greedy;            // what its decision needs, in one 16-byte load
};

struct Header {
  int error;
  int n_rows;
  int n_units;
  int n_stoch;        // stochastic requests (listed in Workspace::stoch_list)
  int n_rows3[3];     // early-exit rounds: rows listed for a round (three lists in rotation)
  int n_res3[3];      // early-exit rounds: residual sweeps listed for a round
  int n_alive3[3];    // early-exit rounds: requests deciding a position in the round
  int n_rows_b;       // rows of the second row list (streamed last)
  int pad[50];
};

struct Workspace {
  Header* hdr;
  ReqInfo* req;
  uint32_t* rowdesc;   // [2K + B]
  uint32_t* rowdesc_b; // [2B]  rows streamed last (position-0 pairs of stochastic requests)
  int* stoch_list;     // [B]   the stochastic requests, in request order
  Partial* pt;         // [(K + B) * nseg]
  Partial* pd;         // [K * nseg]
  double* rp;          // [B * nrseg]
  uint32_t* rows_r;    // [3][2K+B]  early-exit rounds: row descriptors
  int* res_r;          // [3][B]     early-exit rounds: requests whose residual is swept
  int* alive;          // [3][B]     tree rounds: requests still walking
  AliveEntry* alive_e; // [3][B]     early-exit rounds: requests deciding a window
};

struct Args {
  int B, K, V, nseg, seg, nrseg, rseg;
  int force_greedy;
  int64_t tld, dld;
  const void* target;
  const void* draft;
  const int* num_draft;
  const int* tokens;
  const uint8_t* gmask;
  const float* u_accept;
  const float* u_final;
  int* acc_len;
  int* out;
  float* p_out;
  float* q_out;
  float* resid_out;
  float c;            // fl(log2(e)/T): the scale of every exponent
  double c64;         // the same value in fp64
  double T64;         // the fp32 temperature, widened (the fp64 draw divides by it)
  const uint32_t* rowlist;   // rows k_stats reads (all rows, or one round's)
  const int* rowcount;       // number of rows in rowlist
  const uint32_t* rowlist_b = nullptr;   // rows k_stats reads after those, or NULL
  const int* rowcount_b = nullptr;       // number of rows in rowlist_b (when not NULL)
  int plan_in_kernel = 0;    // k_stats plans the call itself (no rowlist; see plan_block)
  int ee_round;              // early-exit round, -1 on the all-rows path
  int ee_lo, ee_hi, ee_nhi;  // early exit: positions [lo, hi) decided in this round, [hi, nhi) in the next
  int max_k;                 // early-exit: bound on every num_draft[b] (trees: on every depth)
  const int* parent;         // token trees: [N] local parent index
  int* path;                 // token trees: [N] walked node indices
  Workspace ws;
};

// ------------------------------------------------------------------ element access
// load():    ordinary 16-byte load (rescans of a single unit, gathers).
// stream():  16-byte nontemporal load for data read once per call; it keeps the
//            streamed logits from displacing other lines and measured faster on
//            gfx950 for read-once sweeps.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct F32 {
  using Elem = float;
  static constexpr int E = 4;
  using Raw = float4;
  __device__ static __forceinline__ Raw load(const Elem* p) {
    return *reinterpret_cast<const float4*>(p);
  }
  __device__ static __forceinline__ Raw stream(const Elem* p) {
    const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return make_float4(t.x, t.y, t.z, t.w);
  }
  __device__ static __forceinline__ void unpack(const Raw& r, float* v) {
    v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
  }
  __device__ static __forceinline__ float one(const Elem* p) { return *p; }
};

struct BF16 {
  using Elem = uint16_t;
  static constexpr int E = 8;
  using Raw = uint4;
  __device__ static __forceinline__ Raw load(const Elem* p) {
    return *reinterpret_cast<const uint4*>(p);
  }
  __device__ static __forceinline__ Raw stream(const Elem* p) {
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
  }
  __device__ static __forceinline__ void unpack(const Raw& r, float* v) {
    v[0] = __uint_as_float(r.x << 16); v[1] = __uint_as_float(r.x & 0xffff0000u);
    v[2] = __uint_as_float(r.y << 16); v[3] = __uint_as_float(r.y & 0xffff0000u);
    v[4] = __uint_as_float(r.z << 16); v[5] = __uint_as_float(r.z & 0xffff0000u);
    v[6] = __uint_as_float(r.w << 16); v[7] = __uint_as_float(r.w & 0xffff0000u);
  }
  __device__ static __forceinline__ float one(const Elem* p) {
    return __uint_as_float(static_cast<uint32_t>(*p) << 16);
  }
};

// Unaligned rows: one element per "chunk", plain scalar loads.
template <class D>
struct Scalar {
  using Elem = typename D::Elem;
  static constexpr int E = 1;
  using Raw = float;
  __device__ static __forceinline__ Raw load(const Elem* p) { return D::one(p); }
  __device__ static __forceinline__ Raw stream(const Elem* p) { return D::one(p); }
  __device__ static __forceinline__ void unpack(const Raw& r, float* v) { v[0] = r; }
  __device__ static __forceinline__ float one(const Elem* p) { return D::one(p); }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// exp((z - m)/T) as exp2((z - m) * c) with the one fp32 scale c = fl(log2(e)/T):
// z - m is exact for bf16 logits (and within half an ulp for f32), the product
// is rounded once, and z <= m keeps the exponent <= 0 for any finite m, so no
// row can overflow.  Every kernel uses this same c, so all of them see the
// softmax at the temperature log2(e)/c (within a relative 2^-24 of T).
__device__ __forceinline__ float scaled_exp(float d, float c) { return fast_exp2(d * c); }

// A softmax row with no mass (every logit -inf) has no distribution; the
// decision kernels report a request that tests such a row as invalid.
__device__ __forceinline__ bool row_has_mass(double S) { return S > 0.0; }

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Visit the unit [s0, s1) of one row, chunk by chunk, in increasing id order
// per lane.  f(v, first_id, count) receives E values (padding = -inf).  The
// loop is software-pipelined: the U chunks of the next step are requested
// before the current U are consumed, so every wavefront keeps loads in flight
// while it computes.  The per-lane order of the chunks does not depend on U,
// so the result is the same bit for bit for any U.
template <class L, int U, class F>
__device__ __forceinline__ void for_unit(const typename L::Elem* row, int s0, int s1,
                                         int lane, F& f) {
  constexpr int E = L::E;
  const int n = s1 - s0;
  const int nchunk = n / E;
  const typename L::Elem* p = row + s0;
  constexpr int per_it = kWave * U;
  const int nit = nchunk / per_it;
  int c = lane;
  auto consume = [&](const typename L::Raw* r) {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      float v[E];
      L::unpack(r[j], v);
      f(v, s0 + (c + j * kWave) * E, E);
    }
  };
  if (nit > 0) {
    typename L::Raw r[U];
#pragma unroll
    for (int j = 0; j < U; ++j) r[j] = L::stream(p + (size_t)(c + j * kWave) * E);
    for (int it = 1; it < nit; ++it) {
      typename L::Raw nx[U];
#pragma unroll
      for (int j = 0; j < U; ++j) nx[j] = L::stream(p + (size_t)(c + per_it + j * kWave) * E);
      consume(r);
#pragma unroll
      for (int j = 0; j < U; ++j) r[j] = nx[j];
      c += per_it;
    }
    consume(r);
    c += per_it;
  }
  for (; c < nchunk; c += kWave) {
    float v[E];
    L::unpack(L::stream(p + (size_t)c * E), v);
    f(v, s0 + c * E, E);
  }
  const int tail0 = nchunk * E;
  if (lane < n - tail0) {
    float v[E];
    v[0] = L::one(p + tail0 + lane);
#pragma unroll
    for (int e = 1; e < E; ++e) v[e] = -INFINITY;
    f(v, s0 + tail0 + lane, 1);
  }
}

template <int E>
struct SoftmaxAcc {
  float m;             // running maximum of the lane
  float s[E];
  float c;
  __device__ __forceinline__ void operator()(const float* v, int, int) {
    float cm = v[0];
#pragma unroll
    for (int e = 1; e < E; ++e) cm = fmaxf(cm, v[e]);
    if (cm > m) {                    // rare after the first chunks
      const float f = scaled_exp(m - cm, c);
#pragma unroll
      for (int e = 0; e < E; ++e) s[e] *= f;
      m = cm;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) s[e] += scaled_exp(v[e] - m, c);
  }
};

template <int E>
struct ArgmaxAcc {
  float best;
  int idx;
  __device__ __forceinline__ void operator()(const float* v, int id0, int cnt) {
    float cm = v[0];
#pragma unroll
    for (int e = 1; e < E; ++e) cm = fmaxf(cm, v[e]);
    if (cm > best) {                 // ids only grow within a lane: strict > keeps the lowest
      int hit = 0;
#pragma unroll
      for (int e = E - 1; e >= 0; --e)
        if (v[e] == cm) hit = e;
      if (hit < cnt) {
        best = cm;
        idx = id0 + hit;
      }
    }
  }
};

template <class L, int U = kUnroll>
__device__ void softmax_unit(const typename L::Elem* row, int s0, int s1, int lane,
                             const Args& a, Partial* out) {
  SoftmaxAcc<L::E> acc;
  acc.m = -FLT_MAX;
  acc.c = a.c;
#pragma unroll
  for (int e = 0; e < L::E; ++e) acc.s[e] = 0.f;
  for_unit<L, U>(row, s0, s1, lane, acc);
  float sl = 0.f;
#pragma unroll
  for (int e = 0; e < L::E; ++e) sl += acc.s[e];
  const float mw = wave_max(acc.m);
  const float f = scaled_exp(acc.m - mw, a.c);
  const double sw = wave_sum((double)sl * (double)f);
  if (lane == 0) {
    Partial p;
    p.s = sw;
    p.m = mw;
    p.idx = 0;
    *out = p;
  }
}

template <class L, int U = kArgmaxUnroll>
__device__ void argmax_unit(const typename L::Elem* row, int s0, int s1, int lane,
                            Partial* out) {
  ArgmaxAcc<L::E> acc;
  acc.best = -INFINITY;
  acc.idx = INT_MAX;
  for_unit<L, U>(row, s0, s1, lane, acc);
  float b = acc.best;
  int i = acc.idx;
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const float ob = __shfl_xor(b, o);
    const int oi = __shfl_xor(i, o);
    if (ob > b || (ob == b && oi < i)) {
      b = ob;
      i = oi;
    }
  }
  if (lane == 0) {
    Partial p;
    p.s = 0.0;
    p.m = b;
    p.idx = i;
    *out = p;
  }
}

// ------------------------------------------------------------------ block scans
__device__ __forceinline__ long long wave_incl_scan_ll(long long x, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const long long y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// Exclusive prefix sums of two 64-bit values over one workgroup of kPlanThreads
// threads, and their totals: wave scans, then wave 0 scans the wave totals.
// Every thread of the workgroup must call it; s0, s1 hold kPlanWaves entries,
// st two.  The caller separates two calls with a barrier.
struct Scan2 {
  long long ex0, ex1, tot0, tot1;
};

__device__ __forceinline__ Scan2 block_scan2(long long v0, long long v1, long long* s0,
                                             long long* s1, long long* st) {
  constexpr int kPlanWaves = kPlanThreads / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  const long long i0 = wave_incl_scan_ll(v0, lane);
  const long long i1 = wave_incl_scan_ll(v1, lane);
  if (lane == kWave - 1) {
    s0[wv] = i0;
    s1[wv] = i1;
  }
  __syncthreads();
  if (wv == 0) {                        // wave totals -> exclusive wave prefixes, in place
    const long long w0 = lane < kPlanWaves ? s0[lane] : 0;
    const long long w1 = lane < kPlanWaves ? s1[lane] : 0;
    const long long c0 = wave_incl_scan_ll(w0, lane);
    const long long c1 = wave_incl_scan_ll(w1, lane);
    if (lane < kPlanWaves) {
      s0[lane] = c0 - w0;
      s1[lane] = c1 - w1;
    }
    if (lane == kPlanWaves - 1) {
      st[0] = c0;
      st[1] = c1;
    }
  }
  __syncthreads();
  Scan2 r;
  r.ex0 = s0[wv] + i0 - v0;
  r.ex1 = s1[wv] + i1 - v1;
  r.tot0 = st[0];
  r.tot1 = st[1];
  return r;
}

// ------------------------------------------------------------------ row lists
// The rows an all-rows call streams, in two lists that k_stats reads in
// order.  The second list holds the position-0 (target, draft) pair of every
// stochastic request with k_b >= 1: about half of all cuts fall at position 0
// and the residual sweep re-reads exactly the rejected pair, so those pairs
// are read last.  The first list holds every other row, request after
// request: all target rows of a greedy request; target rows 1..k_b then draft
// rows 1..k_b-1 of a stochastic request (its target row 0 when k_b = 0).
__device__ __forceinline__ void row_counts(int k, bool g, int& cA, int& cB) {
  const bool pair0 = SV_MALL_ORDER && !g && k >= 1;
  cA = g ? k + 1 : (pair0 ? 2 * k - 1 : 2 * k + 1);
  cB = pair0 ? 2 : 0;
}

// Descriptor of entry j of request b in the first list (off = its offset).
__device__ __forceinline__ uint32_t row_in_first(int b, int j, int off, int k, bool g) {
  if (g) return (uint32_t)(off + b + j) | kGreedyBit;
  const int first = (SV_MALL_ORDER && k >= 1) ? 1 : 0;   // position 0 in the second list
  const int nt = k + 1 - first;                            // target rows of the first list
  return j < nt ? (uint32_t)(off + b + first + j)
                : ((uint32_t)(off + first + (j - nt)) | kDraftBit);
}

// Descriptor of entry j (0: target, 1: draft) of request b in the second list.
__device__ __forceinline__ uint32_t row_in_second(int b, int j, int off) {
  return j == 0 ? (uint32_t)(off + b) : ((uint32_t)off | kDraftBit);
}

// Plan of one call made by every k_stats workgroup when it fits in LDS
// (plan_fits_lds): the exclusive prefix sums over the requests of k_b, of
// their first-list rows and of their second-list rows, and from them the
// table of every row descriptor to stream (first list, then second list), so
// that finding a unit's row is one LDS read.
constexpr int kPlanInKernelMaxB = 2048;     // requests (8 per thread of a workgroup)
constexpr int kPlanInKernelMaxRows = 6144;  // row descriptors (24 KiB of LDS)

__host__ __device__ constexpr bool plan_fits_lds(long long B, long long K) {
  return B <= kPlanInKernelMaxB && 2 * K + B <= kPlanInKernelMaxRows;
}

__host__ __device__ constexpr size_t plan_lds_bytes(long long B, long long K) {
  return (size_t)(2 * K + B) * sizeof(uint32_t);
}

struct Sums4 {
  int k, a, b, s;
};

__device__ __forceinline__ Sums4 wave_incl_scan4(Sums4 x, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int k = __shfl_up(x.k, o), a = __shfl_up(x.a, o);
    const int b = __shfl_up(x.b, o), s = __shfl_up(x.s, o);
    if (lane >= o) {
      x.k += k;
      x.a += a;
      x.b += b;
      x.s += s;
    }
  }
  return x;
}

// Every thread of the k_stats workgroup (kBlock threads) takes part: thread t
// plans the requests [t * per, (t + 1) * per), per = ceil(B / kBlock) <= 8,
// and writes their rows to table (first list at [0, nA), second list at
// [nA, nA + nB)).  Returns false when num_draft is inconsistent (a k_b < 0 or
// > K, or a total other than K); nA, nB are then 0.  records: also write the
// request records, the list of stochastic requests and the header (one
// workgroup does).
__device__ bool plan_block(const Args& a, uint32_t* table, bool records, int& nA, int& nB) {
  __shared__ Sums4 s_w[kWavesPerBlock];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid >> 6;
  const int B = a.B;
  const int per = (B + kBlock - 1) / kBlock;
  const int b0 = tid * per;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  constexpr int kPer = kPlanInKernelMaxB / kBlock;
  int kk[kPer];
  bool gg[kPer];
  Sums4 mine = {0, 0, 0, 0};
  bool bad = false;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    kk[q] = 0;
    gg[q] = true;
    const int b = b0 + q;
    if (q < per && b < B) {
      int k = a.num_draft[b];
      if (k < 0 || k > a.K) {
        bad = true;
        k = 0;
      }
      const bool g = a.force_greedy ? true : (a.gmask ? (a.gmask[b] != 0) : false);
      int cA, cB;
      row_counts(k, g, cA, cB);
      kk[q] = k;
      gg[q] = g;
      mine.k += k;
      mine.a += cA;
      mine.b += cB;
      mine.s += g ? 0 : 1;
    }
  }
  if (bad) s_bad = 1;
  const Sums4 inc = wave_incl_scan4(mine, lane);
  if (lane == kWave - 1) s_w[wv] = inc;
  __syncthreads();
  Sums4 ex = {inc.k - mine.k, inc.a - mine.a, inc.b - mine.b, inc.s - mine.s};
  Sums4 tot = {0, 0, 0, 0};
#pragma unroll
  for (int q = 0; q < kWavesPerBlock; ++q) {
    const Sums4 w = s_w[q];
    if (q < wv) {
      ex.k += w.k;
      ex.a += w.a;
      ex.b += w.b;
      ex.s += w.s;
    }
    tot.k += w.k;
    tot.a += w.a;
    tot.b += w.b;
    tot.s += w.s;
  }
  const bool ok = !s_bad && tot.k == a.K;   // then every table index stays below 2K + B
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int b = b0 + q;
    if (q < per && b < B) {
      int cA, cB;
      row_counts(kk[q], gg[q], cA, cB);
      if (ok) {
        for (int j = 0; j < cA; ++j) table[ex.a + j] = row_in_first(b, j, ex.k, kk[q], gg[q]);
        for (int j = 0; j < cB; ++j) table[tot.a + ex.b + j] = row_in_second(b, j, ex.k);
      }
      if (records) {
        ReqInfo r;
        r.off = ex.k;
        r.k = kk[q];
        r.greedy = gg[q] ? 1 : 0;
        r.a = 0;
        r.kind = KIND_NONE;
        r.y = -1;
        r.trow = -1;
        r.drow = -1;
        r.Mp = r.Mq = 0.f;
        r.pad0 = r.pad1 = 0;
        r.Sp = r.Sq = 0.0;
        a.ws.req[b] = r;
        if (!gg[q]) a.ws.stoch_list[ex.s] = b;
      }
      ex.k += kk[q];
      ex.a += cA;
      ex.b += cB;
      ex.s += gg[q] ? 0 : 1;
    }
  }
  if (records && tid == 0) {
    Header* h = a.ws.hdr;
    h->error = ok ? 0 : 1;
    h->n_rows = ok ? tot.a : 0;
    h->n_rows_b = ok ? tot.b : 0;
    h->n_stoch = ok ? tot.s : 0;
    h->n_units = 0;
  }
  __syncthreads();
  nA = ok ? tot.a : 0;
  nB = ok ? tot.b : 0;
  return ok;
}

// ------------------------------------------------------------------ k_stats
// Persistent grid; wavefront gw takes units gw, gw + W, ...  The rows come
// from the two lists, the first one then the second: from rowlist / rowlist_b
// (written by k_plan), or, when a.plan_in_kernel, from the row table every
// workgroup builds in LDS (dynamic shared memory of plan_lds_bytes(B, K)).
// The descriptor of the next unit is fetched while the current one streams.
template <class L>
__global__ __launch_bounds__(kBlock) void k_stats(Args a) {
  using Elem = typename L::Elem;
  extern __shared__ uint32_t row_table[];
  const int lane = threadIdx.x & (kWave - 1);
  const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int W = gridDim.x * kWavesPerBlock;
  int nA, nB;
  if (a.plan_in_kernel) {
    plan_block(a, row_table, blockIdx.x == 0, nA, nB);
  } else {
    nA = *a.rowcount;
    nB = a.rowcount_b ? *a.rowcount_b : 0;
  }
  const int n_units = (nA + nB) * a.nseg;
  auto desc_of = [&](int ri) -> uint32_t {
    if (a.plan_in_kernel) return row_table[ri];
    return ri < nA ? a.rowlist[ri] : a.rowlist_b[ri - nA];
  };
  const Elem* tgt = static_cast<const Elem*>(a.target);
  const Elem* drf = static_cast<const Elem*>(a.draft);
  uint32_t next = (gw < n_units) ? desc_of(gw / a.nseg) : 0u;
  for (int u = gw; u < n_units; u += W) {
    const uint32_t desc = next;
    const int ri = u / a.nseg;
    const int seg = u - ri * a.nseg;
    if (u + W < n_units) next = desc_of((u + W) / a.nseg);
    const int row = (int)(desc & kRowMask);
    const bool is_draft = (desc & kDraftBit) != 0;
    const bool greedy = (desc & kGreedyBit) != 0;
    const int s0 = seg * a.seg;
    const int s1 = min(s0 + a.seg, a.V);
    const Elem* base = is_draft ? drf + (int64_t)row * a.dld : tgt + (int64_t)row * a.tld;
    Partial* out = (is_draft ? a.ws.pd : a.ws.pt) + (int64_t)row * a.nseg + seg;
    if (greedy)
      argmax_unit<L>(base, s0, s1, lane, out);
    else
      softmax_unit<L>(base, s0, s1, lane, a, out);
  }
}

// ------------------------------------------------------------------ host helpers
size_t align_up(size_t x, size_t al) { return (x + al - 1) / al * al; }

std::atomic<int> g_cu_count[64];

int cu_count(int dev) {
  if (dev >= 0 && dev < 64) {
    const int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int c = 0;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
    c = 256;
  if (dev >= 0 && dev < 64) g_cu_count[dev].store(c, std::memory_order_relaxed);
  return c;
}

// c = fl(log2(e)/T), rounded to nearest; the caller has checked that
// log2(e)/T < FLT_MAX.
void set_scale(double T, float* c, double* c64) {
  *c = (float)(1.4426950408889634 / T);
  *c64 = (double)*c;
}

template <class Kern>
int resident_blocks(std::atomic<int>* cache, Kern kern, int dev) {
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, kBlock, 0) != hipSuccess || n <= 0)
    n = 1;
  n = std::min(n, kBlocksPerCU);
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace
