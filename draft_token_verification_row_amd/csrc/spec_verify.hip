// spec_verify.hip - one-round draft-token verification for AMD Instinct MI355X (gfx950).
//
// Implements the C ABI of include/spec_verify.h.  The operation is the
// verification step of one speculative-decoding round (chzhyang, "Speculative
// Decoding: Medusa, MTP, EAGLE, DFlash, DDTree, and DSpark", section 1; vLLM blog
// "speculative-decoding-amd-gpus", "Core idea of speculative decoding").
//
// All-rows pipeline (spec_verify_greedy / spec_verify_sample; every launch on
// the caller's stream, no host synchronisation):
//   k_plan      one workgroup: exclusive scan of num_draft -> request offsets,
//               compact list of logit rows to read (every target row, the draft
//               rows of stochastic requests), unit count.
//   k_stats     persistent grid, one wavefront per 32 KiB slice ("unit") of a
//               row.  Streams the logits once from HBM with 16-byte loads and
//               writes per-unit partials: online max and sum of exp((z-max)/T)
//               for softmax rows, (max, lowest id) for greedy rows.  This is the
//               HBM-bound kernel that carries almost all bytes.
//   k_decide    one wavefront per request: combines the partials of each row,
//               evaluates p(y_i), q(y_i) in fp64, runs the ratio test (stochastic)
//               or argmax test (greedy) for every position, cuts at the first
//               rejection, commits the kept drafts and the greedy target token,
//               and queues a residual job for stochastic requests cut early.
//   k_resid     persistent grid: second sweep of the one (target, draft) row pair
//               of each queued request, per-unit sums of [p - q]_+.
//   k_finalize  one workgroup per stochastic request: finds the unit holding
//               the inverse-CDF crossing from the unit sums (bonus: from the
//               k_stats partials, no re-read), rescans that unit only and writes
//               the correction / bonus token.
//
// Early-exit pipeline (the *_early_exit entry points): k_plan_ee, then per
// draft position j a k_round launch (row statistics of position j of the
// requests still undecided, residual sweeps of the requests cut at j - 1) and a
// k_decide_round launch (decides position j), then k_finalize.
//
// Numerics.  exp((z - m)/T) is evaluated as exp2((z - m) * c) with
// c = log2(e)/T split into two fp32 constants (c_hi + c_lo), so the rounding of
// c does not bias whole rows.  Lane partial sums are fp32 over at most a few
// dozen terms, combined across lanes, units and rows in fp64.  p(y) and q(y)
// are formed in fp64 from the exact logit at y.  Greedy argmax is exact
// (lexicographic max of (value, -id)).
#include <hip/hip_runtime.h>

#include <float.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "spec_verify.h"

namespace {

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kWavesPerBlock = kBlock / kWave;
#ifndef SV_UNROLL
#define SV_UNROLL 2
#endif
#ifndef SV_SEG_BYTES
#define SV_SEG_BYTES 32768
#endif
constexpr int kUnroll = SV_UNROLL;       // 16-byte loads in flight per lane per row
#ifndef SV_ROUND_UNROLL
#define SV_ROUND_UNROLL 4
#endif
// early-exit rounds: same per-lane chunk order (so the same partials bit for
// bit), more loads in flight for the small late rounds
constexpr int kRoundUnroll = SV_ROUND_UNROLL;
#ifndef SV_RESID_UNROLL
#define SV_RESID_UNROLL 4
#endif
constexpr int kResidUnroll = SV_RESID_UNROLL;   // k_resid: loads in flight per lane per row
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

struct Header {
  int error;
  int n_rows;
  int n_units;
  int n_resid;
  int n_rows3[3];     // early-exit rounds: rows listed for a round (three lists in rotation)
  int n_res3[3];      // early-exit rounds: residual sweeps listed for a round
  int n_alive3[3];    // early-exit rounds: requests deciding a position in the round
  int pad[51];
};

struct Workspace {
  Header* hdr;
  ReqInfo* req;
  uint32_t* rowdesc;   // [2K + B]
  int* resid_list;     // [B]
  Partial* pt;         // [(K + B) * nseg]
  Partial* pd;         // [K * nseg]
  double* rp;          // [B * nrseg]
  uint32_t* rows_r;    // [3][2B]    early-exit rounds: row descriptors
  int* res_r;          // [3][B]     early-exit rounds: requests whose residual is swept
  int* alive;          // [3][B]     early-exit rounds: requests deciding a position
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
  float c_hi, c_lo;    // log2(e)/T split into two fp32 constants, c_lo > 0
  double c64, T64;
  const uint32_t* rowlist;   // rows k_stats reads (all rows, or one round's)
  const int* rowcount;       // number of rows in rowlist
  int ee_round;              // early-exit round, -1 on the all-rows path
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

// exp((z - m)/T) = exp2(d * c) with d = z - m and c = c_hi + c_lo.
__device__ __forceinline__ float scaled_exp(float d, float c_hi, float c_lo) {
  return fast_exp2(fmaf(d, c_hi, d * c_lo));
}

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
// per lane.  f(v, first_id, count) receives E values (padding = -inf).
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
  for (int it = 0; it < nit; ++it, c += per_it) {
    typename L::Raw r[U];
#pragma unroll
    for (int j = 0; j < U; ++j) r[j] = L::stream(p + (size_t)(c + j * kWave) * E);
#pragma unroll
    for (int j = 0; j < U; ++j) {
      float v[E];
      L::unpack(r[j], v);
      f(v, s0 + (c + j * kWave) * E, E);
    }
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
  float m;
  float s[E];
  float c_hi, c_lo;
  __device__ __forceinline__ void operator()(const float* v, int, int) {
    float cm = v[0];
#pragma unroll
    for (int e = 1; e < E; ++e) cm = fmaxf(cm, v[e]);
    if (cm > m) {                    // rare after the first chunks
      const float f = scaled_exp(m - cm, c_hi, c_lo);
#pragma unroll
      for (int e = 0; e < E; ++e) s[e] *= f;
      m = cm;
    }
#pragma unroll
    for (int e = 0; e < E; ++e) s[e] += scaled_exp(v[e] - m, c_hi, c_lo);
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
  acc.c_hi = a.c_hi;
  acc.c_lo = a.c_lo;
#pragma unroll
  for (int e = 0; e < L::E; ++e) acc.s[e] = 0.f;
  for_unit<L, U>(row, s0, s1, lane, acc);
  float sl = 0.f;
#pragma unroll
  for (int e = 0; e < L::E; ++e) sl += acc.s[e];
  const float mw = wave_max(acc.m);
  const float f = scaled_exp(acc.m - mw, a.c_hi, a.c_lo);
  const double sw = wave_sum((double)sl * (double)f);
  if (lane == 0) {
    Partial p;
    p.s = sw;
    p.m = mw;
    p.idx = 0;
    *out = p;
  }
}

template <class L, int U = kUnroll>
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

// ------------------------------------------------------------------ k_plan
__device__ __forceinline__ long long wave_incl_scan_ll(long long x, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const long long y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// One workgroup: exclusive scans of k_b (all requests) and of k_b over
// stochastic requests, 1024 requests per pass (wave shuffles + one LDS step).
__global__ __launch_bounds__(kPlanThreads) void k_plan(Args a) {
  constexpr int kPlanWaves = kPlanThreads / kWave;
  __shared__ long long s_wk[kPlanWaves];
  __shared__ long long s_ws[kPlanWaves];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid >> 6;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  const long long TB = (long long)a.K + a.B;
  long long carry_k = 0, carry_s = 0;
  for (int base = 0; base < a.B; base += kPlanThreads) {
    const int b = base + tid;
    long long k = 0;
    int g = 1;
    if (b < a.B) {
      int kk = a.num_draft[b];
      if (kk < 0 || kk > a.K) {
        s_bad = 1;
        kk = 0;
      }
      k = kk;
      g = a.force_greedy ? 1 : (a.gmask ? (a.gmask[b] != 0) : 0);
    }
    const long long ks = g ? 0 : k;
    const long long ik = wave_incl_scan_ll(k, lane);
    const long long is = wave_incl_scan_ll(ks, lane);
    if (lane == kWave - 1) {
      s_wk[wv] = ik;
      s_ws[wv] = is;
    }
    __syncthreads();
    long long pk = 0, ps = 0, tot_k = 0, tot_s = 0;
    for (int q = 0; q < kPlanWaves; ++q) {
      if (q < wv) {
        pk += s_wk[q];
        ps += s_ws[q];
      }
      tot_k += s_wk[q];
      tot_s += s_ws[q];
    }
    const long long off = carry_k + pk + ik - k;
    const long long soff = carry_s + ps + is - ks;
    if (b < a.B) {
      ReqInfo r;
      r.off = (int)off;
      r.k = (int)k;
      r.greedy = g;
      r.a = 0;
      r.kind = KIND_NONE;
      r.y = -1;
      r.trow = -1;
      r.drow = -1;
      r.Mp = r.Mq = 0.f;
      r.pad0 = r.pad1 = 0;
      r.Sp = r.Sq = 0.0;
      a.ws.req[b] = r;
      for (long long i = 0; i <= k; ++i) {
        const long long row = off + b + i;
        if (row < TB) a.ws.rowdesc[row] = (uint32_t)row | (g ? kGreedyBit : 0u);
      }
      if (!g) {
        for (long long i = 0; i < k; ++i) {
          const long long slot = TB + soff + i;
          if (slot < TB + a.K) a.ws.rowdesc[slot] = (uint32_t)(off + i) | kDraftBit;
        }
      }
    }
    carry_k += tot_k;
    carry_s += tot_s;
    __syncthreads();
  }
  if (tid == 0) {
    const bool bad = s_bad != 0 || carry_k != a.K;
    const long long nrows = bad ? 0 : TB + carry_s;
    Header* h = a.ws.hdr;
    h->error = bad ? 1 : 0;
    h->n_rows = (int)nrows;
    h->n_units = (int)(nrows * a.nseg);
    h->n_resid = 0;
  }
}

// ------------------------------------------------------------------ k_stats
// Persistent grid; wavefront gw takes units gw, gw + W, ...  The descriptor of
// the next unit is fetched while the current one streams.
template <class L>
__global__ __launch_bounds__(kBlock) void k_stats(Args a) {
  using Elem = typename L::Elem;
  const int lane = threadIdx.x & (kWave - 1);
  const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int W = gridDim.x * kWavesPerBlock;
  const int n_units = *a.rowcount * a.nseg;
  const Elem* tgt = static_cast<const Elem*>(a.target);
  const Elem* drf = static_cast<const Elem*>(a.draft);
  uint32_t next = (gw < n_units) ? a.rowlist[gw / a.nseg] : 0u;
  for (int u = gw; u < n_units; u += W) {
    const uint32_t desc = next;
    const int ri = u / a.nseg;
    const int seg = u - ri * a.nseg;
    if (u + W < n_units) next = a.rowlist[(u + W) / a.nseg];
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

// ------------------------------------------------------------------ row combines
// One lane combines the nseg unit partials of one row.  Loads are issued in
// groups of 16 so that they are in flight together (one group covers a
// 262144-id bf16 row); unit factors use the same split-constant exp2 as the
// streaming kernels and accumulate in fp64.
constexpr int kCombineGroup = 16;

__device__ void row_softmax(const Partial* P, int nseg, float c_hi, float c_lo, float& M,
                            double& S) {
  float m = -FLT_MAX;
  double s = 0.0;
  for (int g0 = 0; g0 < nseg; g0 += kCombineGroup) {
    float pm[kCombineGroup];
    double ps[kCombineGroup];
#pragma unroll
    for (int j = 0; j < kCombineGroup; ++j) {
      if (g0 + j < nseg) {
        const Partial p = P[g0 + j];
        pm[j] = p.m;
        ps[j] = p.s;
      } else {
        pm[j] = -FLT_MAX;
        ps[j] = 0.0;
      }
    }
    float gm = m;
#pragma unroll
    for (int j = 0; j < kCombineGroup; ++j) gm = fmaxf(gm, pm[j]);
    if (gm > m) {
      s *= (double)scaled_exp(m - gm, c_hi, c_lo);
      m = gm;
    }
#pragma unroll
    for (int j = 0; j < kCombineGroup; ++j)
      if (ps[j] > 0.0) s += ps[j] * (double)scaled_exp(pm[j] - m, c_hi, c_lo);
  }
  M = m;
  S = s;
}

__device__ void row_argmax(const Partial* P, int nseg, int& idx) {
  float bm = -INFINITY;
  int bi = INT_MAX;
  for (int g0 = 0; g0 < nseg; g0 += kCombineGroup) {
    float pm[kCombineGroup];
    int pi[kCombineGroup];
#pragma unroll
    for (int j = 0; j < kCombineGroup; ++j) {
      if (g0 + j < nseg) {
        const Partial p = P[g0 + j];
        pm[j] = p.m;
        pi[j] = p.idx;
      } else {
        pm[j] = -INFINITY;
        pi[j] = INT_MAX;
      }
    }
#pragma unroll
    for (int j = 0; j < kCombineGroup; ++j) {
      if (pm[j] > bm || (pm[j] == bm && pi[j] < bi)) {
        bm = pm[j];
        bi = pi[j];
      }
    }
  }
  idx = bi;
}

template <class D>
__device__ __forceinline__ float logit_at(const void* base, int64_t row, int64_t ld, int v) {
  return D::one(static_cast<const typename D::Elem*>(base) + row * ld + v);
}

// ------------------------------------------------------------------ k_decide
// One wavefront per request.  Positions are taken 32 at a time: lane l < 32
// combines the target row of position base+l, lane l+32 the draft row of the
// same position, so every row of a request is combined in parallel.
// Decision of every position of request b by one wavefront (all rows' partials
// are in the workspace).  queue: list the request for k_resid when it needs a
// residual sweep (the single-launch path sweeps it in the same workgroup).
template <class D>
__device__ void decide_request(const Args& a, int b, int lane, bool queue) {
  const ReqInfo R = a.ws.req[b];
  const int k = R.k;
  const int trow0 = R.off + b;
  const int drow0 = R.off;
  const bool g = R.greedy != 0;
  const int nseg = a.nseg;
  const int half = lane & 31;
  const bool upper = lane >= 32;
  int A = k;
  bool found = false;       // A fixed (a rejection seen, or the bonus row reached)
  bool invalid = false;
  float MpA = 0.f, MqA = 0.f;
  double SpA = 0.0, SqA = 0.0;
  int amaxA = INT_MAX;
  for (int base = 0; base <= k; base += 32) {
    const int i = base + half;
    // issue the gathers at y first; they do not depend on the row statistics
    int y = 0;
    bool yok = false;
    float zy = 0.f, dy = 0.f;
    if (!upper && i < k) {
      y = a.tokens[drow0 + i];
      yok = (y >= 0 && y < a.V);
      if (!g && yok) {
        zy = logit_at<D>(a.target, trow0 + i, a.tld, y);
        dy = logit_at<D>(a.draft, drow0 + i, a.dld, y);
      }
    }
    float M = 0.f;
    double S = 0.0;
    int amax = INT_MAX;
    if (!upper && i <= k) {
      const Partial* P = a.ws.pt + (int64_t)(trow0 + i) * nseg;
      if (g)
        row_argmax(P, nseg, amax);
      else
        row_softmax(P, nseg, a.c_hi, a.c_lo, M, S);
    } else if (upper && !g && i < k) {
      row_softmax(a.ws.pd + (int64_t)(drow0 + i) * nseg, nseg, a.c_hi, a.c_lo, M, S);
    }
    const float Mq = __shfl(M, half + 32);
    const double Sq = __shfl(S, half + 32);
    bool rej = false;
    if (!upper && i < k) {
      if (g) {
        rej = (y != amax);
        if (a.p_out) a.p_out[drow0 + i] = -1.f;   // no probabilities for greedy rows
        if (a.q_out) a.q_out[drow0 + i] = -1.f;
      } else if (!yok) {
        invalid = true;
        if (a.p_out) a.p_out[drow0 + i] = -1.f;
        if (a.q_out) a.q_out[drow0 + i] = -1.f;
      } else {
        const double py = exp(((double)zy - (double)M) / a.T64) / S;
        const double qy = exp(((double)dy - (double)Mq) / a.T64) / Sq;
        rej = !((double)a.u_accept[drow0 + i] * qy < py);
        if (a.p_out) a.p_out[drow0 + i] = (float)py;
        if (a.q_out) a.q_out[drow0 + i] = (float)qy;
      }
    }
    const unsigned long long rm = __ballot(rej);
    if (!found && rm != 0ull) {
      A = base + __ffsll((long long)rm) - 1;
      found = true;
    } else if (!found && k < base + 32) {
      found = true;      // A = k, the bonus row lies in this chunk
    }
    if (found && A >= base && A < base + 32) {
      const int src = A - base;
      MpA = __shfl(M, src);
      SpA = __shfl(S, src);
      MqA = __shfl(M, src + 32);
      SqA = __shfl(S, src + 32);
      amaxA = __shfl(amax, src);
    }
    if (g && found) break;
  }
  if (__any(invalid)) {
    for (int i = lane; i <= k; i += kWave) a.out[trow0 + i] = -1;
    if (lane == 0) {
      a.acc_len[b] = -1;
      if (a.resid_out) a.resid_out[b] = -1.f;
      a.ws.req[b].kind = KIND_INVALID;
    }
    return;
  }
  const int final_tok = g ? (amaxA == INT_MAX ? -1 : amaxA) : -1;
  for (int i = lane; i <= k; i += kWave) {
    int v = -1;
    if (i < A) v = a.tokens[drow0 + i];
    else if (i == A) v = final_tok;     // stochastic: written by k_finalize
    a.out[trow0 + i] = v;
  }
  if (lane == 0) {
    a.acc_len[b] = A;
    if (a.resid_out) a.resid_out[b] = -1.f;
    ReqInfo W = R;
    W.a = A;
    W.trow = trow0 + A;
    if (g) {
      W.kind = KIND_NONE;
    } else {
      W.Mp = MpA;
      W.Sp = SpA;
      if (A < k) {
        W.kind = KIND_RESID;
        W.drow = drow0 + A;
        W.y = a.tokens[drow0 + A];
        W.Mq = MqA;
        W.Sq = SqA;
        if (queue) {
          const int j = atomicAdd(&a.ws.hdr->n_resid, 1);
          a.ws.resid_list[j] = b;
        }
      } else {
        W.kind = KIND_BONUS;
        W.drow = -1;
        W.y = -1;
      }
    }
    a.ws.req[b] = W;
  }
}


template <class D>
__global__ __launch_bounds__(kBlock) void k_decide(Args a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int b = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (a.ws.hdr->error) {
    // inconsistent num_draft: every output slot becomes -1
    const long long gt = (long long)blockIdx.x * kBlock + threadIdx.x;
    const long long gs = (long long)gridDim.x * kBlock;
    for (long long i = gt; i < (long long)a.K + a.B; i += gs) a.out[i] = -1;
    for (long long i = gt; i < a.B; i += gs) {
      a.acc_len[i] = -1;
      if (a.resid_out) a.resid_out[i] = -1.f;
    }
    for (long long i = gt; i < a.K; i += gs) {
      if (a.p_out) a.p_out[i] = -1.f;
      if (a.q_out) a.q_out[i] = -1.f;
    }
    return;
  }
  if (b >= a.B) return;
  decide_request<D>(a, b, lane, true);
}

// ------------------------------------------------------------------ draw weights
// Residual weight [p - q]_+ and target weight p of one id, from the exact row
// maxima and fp32 reciprocals of the row sums.  k_resid and k_finalize use
// these same functions, so both see identical per-id values.
struct ResidW {
  float Mp, Mq, ip, iq, c_hi, c_lo;
  __device__ __forceinline__ float operator()(float z, float d) const {
    const float p = scaled_exp(z - Mp, c_hi, c_lo) * ip;
    const float q = scaled_exp(d - Mq, c_hi, c_lo) * iq;
    return fmaxf(p - q, 0.f);
  }
};

struct TargetW {
  float Mp, ip, c_hi, c_lo;
  __device__ __forceinline__ float operator()(float z) const {
    return scaled_exp(z - Mp, c_hi, c_lo) * ip;
  }
};

__device__ __forceinline__ ResidW resid_weights(const ReqInfo& R, const Args& a) {
  ResidW w;
  w.Mp = R.Mp;
  w.Mq = R.Mq;
  w.ip = (float)(1.0 / R.Sp);
  w.iq = (float)(1.0 / R.Sq);
  w.c_hi = a.c_hi;
  w.c_lo = a.c_lo;
  return w;
}

__device__ __forceinline__ TargetW target_weights(const ReqInfo& R, const Args& a) {
  TargetW w;
  w.Mp = R.Mp;
  w.ip = (float)(1.0 / R.Sp);
  w.c_hi = a.c_hi;
  w.c_lo = a.c_lo;
  return w;
}

// Sum of [p - q]_+ over the ids [s0, s1) of one (target, draft) row pair, the
// rejected id y excluded; one wavefront, result in every lane.
template <class L, int U>
__device__ __forceinline__ double resid_unit(const typename L::Elem* tp, const typename L::Elem* dp,
                                             const ResidW& fw, int y, int s0, int s1, int lane) {
  constexpr int E = L::E;
  const int n = s1 - s0;
  const int nchunk = n / E;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  auto chunk = [&](const typename L::Raw& rt, const typename L::Raw& rd, int id0) {
    float vt[E], vd[E];
    L::unpack(rt, vt);
    L::unpack(rd, vd);
    float r[E];
#pragma unroll
    for (int e = 0; e < E; ++e) r[e] = fw(vt[e], vd[e]);
    if ((unsigned)(y - id0) < (unsigned)E) {
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (id0 + e == y) r[e] = 0.f;   // reject => p(y) < q(y) => [p - q]_+ is 0 at y
    }
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += r[e];
  };
  constexpr int per_it = kWave * U;
  const int nit = nchunk / per_it;
  int c = lane;
  for (int it = 0; it < nit; ++it, c += per_it) {
    typename L::Raw rt[U], rd[U];
#pragma unroll
    for (int jj = 0; jj < U; ++jj) {
      rt[jj] = L::stream(tp + s0 + (size_t)(c + jj * kWave) * E);
      rd[jj] = L::stream(dp + s0 + (size_t)(c + jj * kWave) * E);
    }
#pragma unroll
    for (int jj = 0; jj < U; ++jj) chunk(rt[jj], rd[jj], s0 + (c + jj * kWave) * E);
  }
  for (; c < nchunk; c += kWave)
    chunk(L::stream(tp + s0 + (size_t)c * E), L::stream(dp + s0 + (size_t)c * E), s0 + c * E);
  const int tail0 = nchunk * E;
  if (lane < n - tail0) {
    const int v = s0 + tail0 + lane;
    if (v != y) acc[0] += fw(L::one(tp + v), L::one(dp + v));
  }
  float sl = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) sl += acc[e];
  return wave_sum((double)sl);
}

// ------------------------------------------------------------------ k_resid
// Persistent grid; one wavefront per residual unit (rseg ids of one row pair).
template <class L>
__global__ __launch_bounds__(kBlock) void k_resid(Args a) {
  using Elem = typename L::Elem;
  const int lane = threadIdx.x & (kWave - 1);
  const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int W = gridDim.x * kWavesPerBlock;
  // each wavefront takes a contiguous range of units, so consecutive units
  // mostly share a request and its record is fetched once
  const long long n_units = (long long)a.ws.hdr->n_resid * a.nrseg;
  const int u_begin = (int)(n_units * gw / W);
  const int u_end = (int)(n_units * (gw + 1) / W);
  int cur = -1, b = 0;
  ReqInfo R;
  ResidW fw;
  const Elem* tp = nullptr;
  const Elem* dp = nullptr;
  for (int u = u_begin; u < u_end; ++u) {
    const int j = u / a.nrseg;
    const int seg = u - j * a.nrseg;
    if (j != cur) {
      cur = j;
      b = a.ws.resid_list[j];
      R = a.ws.req[b];
      fw = resid_weights(R, a);
      tp = static_cast<const Elem*>(a.target) + (int64_t)R.trow * a.tld;
      dp = static_cast<const Elem*>(a.draft) + (int64_t)R.drow * a.dld;
    }
    const int s0 = seg * a.rseg;
    const int s1 = min(s0 + a.rseg, a.V);
    const double tot = resid_unit<L, kResidUnroll>(tp, dp, fw, R.y, s0, s1, lane);
    if (lane == 0) a.ws.rp[(int64_t)b * a.nrseg + seg] = tot;
  }
}

// ------------------------------------------------------------------ k_finalize
__device__ __forceinline__ double wave_incl_scan(double x, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const double y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// Mass of unit s for the draw: residual unit sums, or target mass of a
// k_stats unit (its partial rescaled to the row maximum and sum).
struct UnitMass {
  const double* rp;
  const Partial* prow;
  float Mp, c_hi, c_lo;
  double invSp;
  bool resid;
  __device__ __forceinline__ double operator()(int s) const {
    if (resid) return rp[s];
    const Partial p = prow[s];
    return p.s > 0.0 ? p.s * (double)scaled_exp(p.m - Mp, c_hi, c_lo) * invSp : 0.0;
  }
};

// Wave 0 finds the unit holding the crossing of w * Z.  Returns (in lane 0's
// view, broadcast) the unit, the cumulative mass before it and a fallback flag.
__device__ void find_unit(const UnitMass& um, int nunits, double w, int lane, double& Z,
                          int& unit, double& before, int& fallback) {
  // Z is the total of the same chunked scan that locates the crossing, so the
  // two agree bit for bit; with <= 64 units (the usual case) masses load once.
  double m0 = (lane < nunits) ? um(lane) : 0.0;
  double tot = 0.0;
  for (int c0 = 0; c0 < nunits; c0 += kWave) {
    const double m = (c0 == 0) ? m0 : ((c0 + lane < nunits) ? um(c0 + lane) : 0.0);
    tot = __shfl(tot + wave_incl_scan(m, lane), kWave - 1);
  }
  Z = tot;
  const double thr = w * Z;
  double carry = 0.0;
  unit = -1;
  int last_pos = -1;
  double last_before = 0.0;
  for (int c0 = 0; c0 < nunits && unit < 0; c0 += kWave) {
    const double m = (c0 == 0) ? m0 : ((c0 + lane < nunits) ? um(c0 + lane) : 0.0);
    const double incl = carry + wave_incl_scan(m, lane);
    const double excl = incl - m;
    const unsigned long long hit = __ballot(incl > thr && m > 0.0);
    const unsigned long long pos = __ballot(m > 0.0);
    if (hit) {
      const int src = __ffsll((long long)hit) - 1;
      unit = c0 + src;
      before = __shfl(excl, src);
    } else if (pos) {
      const int src = 63 - __clzll((long long)pos);
      last_pos = c0 + src;
      last_before = __shfl(excl, src);
    }
    carry = __shfl(incl, kWave - 1);
  }
  fallback = 0;
  if (unit < 0) {      // rounding left w * Z at or past the end
    unit = last_pos < 0 ? 0 : last_pos;
    before = last_before;
    fallback = 1;
  }
}

// Weights of the ids [id0, id0 + E) of a unit ending at s1 (0 past s1 and at y).
template <class L, class WF>
__device__ __forceinline__ void unit_weights(const typename L::Elem* tp, const typename L::Elem* dp,
                                             int id0, int s1, int y, const WF& wf, float* w) {
  constexpr int E = L::E;
  float vt[E], vd[E];
  if (id0 + E <= s1) {
    L::unpack(L::load(tp + id0), vt);
    if (dp) L::unpack(L::load(dp + id0), vd);
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      vt[e] = (id0 + e < s1) ? L::one(tp + id0 + e) : -INFINITY;
      vd[e] = (dp && id0 + e < s1) ? L::one(dp + id0 + e) : 0.f;
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    float x;
    if constexpr (std::is_same<WF, ResidW>::value) x = wf(vt[e], vd[e]);
    else x = wf(vt[e]);
    w[e] = (id0 + e < s1 && id0 + e != y) ? x : 0.f;
  }
}

// Rescan one unit of PER * kBlock ids: thread t (< kBlock) sums the weights of
// its PER ids in ascending order, a block-wide exclusive scan of those sums
// locates the crossing thread, which walks its ids again.  KEEP holds the
// weights in registers for that walk; otherwise they are recomputed (same
// values, fewer registers).  In a block larger than kBlock the extra threads
// take part in the barriers only, so the result is the same for any block size.
template <class L, int PER, bool KEEP, class WF>
__device__ int rescan_unit(const typename L::Elem* tp, const typename L::Elem* dp, int s0,
                           int s1, int y, const WF& wf, double before, double thr, int fallback,
                           double* s_wave, int* s_owner) {
  constexpr int E = L::E;
  static_assert(PER % E == 0, "per-thread ids must be whole chunks");
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid >> 6;
  const bool active = tid < kBlock;
  const int v0 = s0 + tid * PER;
  float keep[KEEP ? PER : 1];
  double ts = 0.0;
  if (active) {
#pragma unroll
    for (int c = 0; c < PER / E; ++c) {
      float w[E];
      unit_weights<L>(tp, dp, v0 + c * E, s1, y, wf, w);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        ts += (double)w[e];
        if constexpr (KEEP) keep[c * E + e] = w[e];
      }
    }
  }
  // weights of chunk c for the walks below
  auto chunk = [&](int c, float* w) {
    if constexpr (KEEP) {
#pragma unroll
      for (int e = 0; e < E; ++e) w[e] = keep[c * E + e];
    } else {
      unit_weights<L>(tp, dp, v0 + c * E, s1, y, wf, w);
    }
  };
  const double incl_w = wave_incl_scan(ts, lane);
  if (active && lane == kWave - 1) s_wave[wv] = incl_w;
  if (tid == 0) *s_owner = INT_MAX;
  __syncthreads();
  double wprefix = 0.0;
  if (active)
    for (int q = 0; q < wv; ++q) wprefix += s_wave[q];
  const double prev = __shfl_up(incl_w, 1);
  const double excl = before + wprefix + (lane == 0 ? 0.0 : prev);
  const double incl = before + wprefix + incl_w;
  if (active && !fallback && incl > thr && ts > 0.0) atomicMin(s_owner, tid);
  __syncthreads();
  int owner = *s_owner;
  if (owner == INT_MAX) {
    // no thread crosses (rounding, or w*Z past the end): last thread with mass
    __syncthreads();
    if (tid == 0) *s_owner = -1;
    __syncthreads();
    if (active && ts > 0.0) atomicMax(s_owner, tid);
    __syncthreads();
    owner = *s_owner;
    if (tid == owner) {
      int tok = -1;
#pragma unroll
      for (int c = 0; c < PER / E; ++c) {
        float w[E];
        chunk(c, w);
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (w[e] > 0.f) tok = v0 + c * E + e;
      }
      return tok;
    }
    return -2;
  }
  if (tid != owner) return -2;
  double cum = excl;
  int tok = -1, last = -1;
#pragma unroll
  for (int c = 0; c < PER / E; ++c) {
    float w[E];
    chunk(c, w);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      cum += (double)w[e];
      if (w[e] > 0.f) last = v0 + c * E + e;
      if (tok < 0 && cum > thr) tok = v0 + c * E + e;
    }
  }
  return tok >= 0 ? tok : last;
}

struct FinalizeShared {
  double wave[kWavesPerBlock];
  double before, thr, Z;
  int unit, mode, fallback, owner;
};

// Correction or bonus draw of request b by one block of >= kBlock threads
// (KEEP: see rescan_unit).
template <class L, bool KEEP>
__device__ void finalize_request(const Args& a, int b, FinalizeShared& sh) {
  using Elem = typename L::Elem;
  constexpr int PER_S = kSegBytes / (int)sizeof(Elem) / kBlock;    // k_stats unit
  constexpr int PER_R = kRSegBytes / (int)sizeof(Elem) / kBlock;   // k_resid unit
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const ReqInfo R = a.ws.req[b];
  if (R.kind != KIND_RESID && R.kind != KIND_BONUS) return;
  const double w = (double)a.u_final[b];
  if (tid < kWave) {
    UnitMass um;
    um.rp = a.ws.rp + (int64_t)b * a.nrseg;
    um.prow = a.ws.pt + (int64_t)R.trow * a.nseg;
    um.Mp = R.Mp;
    um.c_hi = a.c_hi;
    um.c_lo = a.c_lo;
    um.invSp = 1.0 / R.Sp;
    um.resid = (R.kind == KIND_RESID);
    int mode = um.resid ? DRAW_RESID : DRAW_FROM_P;
    double Z = 0.0, before = 0.0;
    int unit = 0, fb = 0;
    find_unit(um, um.resid ? a.nrseg : a.nseg, w, lane, Z, unit, before, fb);
    if (mode == DRAW_RESID && !(Z > 0.0)) {     // p == q numerically: draw from p
      mode = DRAW_FROM_P;
      um.resid = false;
      find_unit(um, a.nseg, w, lane, Z, unit, before, fb);
    }
    if (tid == 0) {
      sh.unit = unit;
      sh.before = before;
      sh.thr = w * Z;
      sh.Z = Z;
      sh.mode = mode;
      sh.fallback = fb;
    }
  }
  __syncthreads();
  const int mode = sh.mode;
  const Elem* tp = static_cast<const Elem*>(a.target) + (int64_t)R.trow * a.tld;
  int tok;
  if (mode == DRAW_RESID) {
    const Elem* dp = static_cast<const Elem*>(a.draft) + (int64_t)R.drow * a.dld;
    const int s0 = sh.unit * a.rseg;
    const int s1 = min(s0 + a.rseg, a.V);
    tok = rescan_unit<L, PER_R, KEEP>(tp, dp, s0, s1, R.y, resid_weights(R, a), sh.before,
                                      sh.thr, sh.fallback, sh.wave, &sh.owner);
  } else {
    const int s0 = sh.unit * a.seg;
    const int s1 = min(s0 + a.seg, a.V);
    tok = rescan_unit<L, PER_S, KEEP>(tp, (const Elem*)nullptr, s0, s1, -1,
                                      target_weights(R, a), sh.before, sh.thr, sh.fallback,
                                      sh.wave, &sh.owner);
  }
  if (tok != -2) {
    a.out[R.trow] = tok;
    if (a.resid_out)
      a.resid_out[b] = (R.kind == KIND_RESID) ? (float)(mode == DRAW_RESID ? sh.Z : 0.0) : -1.f;
  }
}

template <class L>
__global__ __launch_bounds__(kBlock) void k_finalize(Args a) {
  __shared__ FinalizeShared sh;
  if (a.ws.hdr->error) return;
  finalize_request<L, true>(a, blockIdx.x, sh);
}

// ------------------------------------------------------------------ single-launch path
// Small batches: one workgroup of kFusedThreads threads per request runs the
// whole step (offsets, row statistics, decisions, residual sweep, draw) with
// only block barriers between the phases, so a call is one launch instead of
// five.  Every phase calls the same unit, combine, decide and draw code as the
// multi-kernel path, so the results are the same bit for bit.
constexpr int kFusedThreads = 1024;
constexpr int kFusedWaves = kFusedThreads / kWave;
constexpr int kFusedUnroll = 8;

template <class L>
__global__ __launch_bounds__(kFusedThreads) void k_fused(Args a) {
  __shared__ FinalizeShared sh;
  __shared__ long long s_pre[kFusedWaves], s_tot[kFusedWaves];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid >> 6;
  const int b = blockIdx.x;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  // offsets: every workgroup sums num_draft itself (B is small on this path)
  long long pre = 0, tot = 0;
  for (int i = tid; i < a.B; i += kFusedThreads) {
    const int k = a.num_draft[i];
    if (k < 0 || k > a.K) s_bad = 1;
    else {
      tot += k;
      if (i < b) pre += k;
    }
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    pre += __shfl_xor(pre, o);
    tot += __shfl_xor(tot, o);
  }
  if (lane == 0) {
    s_pre[wv] = pre;
    s_tot[wv] = tot;
  }
  __syncthreads();
  pre = 0;
  tot = 0;
  for (int q = 0; q < kFusedWaves; ++q) {
    pre += s_pre[q];
    tot += s_tot[q];
  }
  if (s_bad || tot != a.K) {
    // inconsistent num_draft: this workgroup clears its share of every output
    const long long gt = (long long)b * kFusedThreads + tid;
    const long long gs = (long long)a.B * kFusedThreads;
    for (long long i = gt; i < (long long)a.K + a.B; i += gs) a.out[i] = -1;
    for (long long i = gt; i < a.K; i += gs) {
      if (a.p_out) a.p_out[i] = -1.f;
      if (a.q_out) a.q_out[i] = -1.f;
    }
    if (tid == 0) {
      a.acc_len[b] = -1;
      if (a.resid_out) a.resid_out[b] = -1.f;
    }
    return;
  }
  const int k = a.num_draft[b];
  const int g = a.force_greedy ? 1 : (a.gmask ? (a.gmask[b] != 0) : 0);
  const int off = (int)pre;
  if (tid == 0) {
    ReqInfo r;
    r.off = off;
    r.k = k;
    r.greedy = g;
    r.a = 0;
    r.kind = KIND_NONE;
    r.y = -1;
    r.trow = -1;
    r.drow = -1;
    r.Mp = r.Mq = 0.f;
    r.pad0 = r.pad1 = 0;
    r.Sp = r.Sq = 0.0;
    a.ws.req[b] = r;
  }
  // row statistics: k + 1 target rows, then the k draft rows of a stochastic request
  using Elem = typename L::Elem;
  const Elem* tgt = static_cast<const Elem*>(a.target);
  const Elem* drf = static_cast<const Elem*>(a.draft);
  const int n_rows = k + 1 + (g ? 0 : k);
  const int n_units = n_rows * a.nseg;
  for (int u = wv; u < n_units; u += kFusedWaves) {
    const int r = u / a.nseg;
    const int seg = u - r * a.nseg;
    const bool is_draft = r > k;
    const int row = is_draft ? off + (r - k - 1) : off + b + r;
    const int s0 = seg * a.seg;
    const int s1 = min(s0 + a.seg, a.V);
    const Elem* base = is_draft ? drf + (int64_t)row * a.dld : tgt + (int64_t)row * a.tld;
    Partial* out = (is_draft ? a.ws.pd : a.ws.pt) + (int64_t)row * a.nseg + seg;
    if (g)
      argmax_unit<L, kFusedUnroll>(base, s0, s1, lane, out);
    else
      softmax_unit<L, kFusedUnroll>(base, s0, s1, lane, a, out);
  }
  __syncthreads();
  if (wv == 0) decide_request<L>(a, b, lane, false);
  __syncthreads();
  const ReqInfo R = a.ws.req[b];
  if (R.kind == KIND_RESID) {
    const Elem* tp = tgt + (int64_t)R.trow * a.tld;
    const Elem* dp = drf + (int64_t)R.drow * a.dld;
    const ResidW fw = resid_weights(R, a);
    for (int seg = wv; seg < a.nrseg; seg += kFusedWaves) {
      const int s0 = seg * a.rseg;
      const int s1 = min(s0 + a.rseg, a.V);
      const double t = resid_unit<L, kFusedUnroll>(tp, dp, fw, R.y, s0, s1, lane);
      if (lane == 0) a.ws.rp[(int64_t)b * a.nrseg + seg] = t;
    }
    __syncthreads();
  }
  finalize_request<L, false>(a, b, sh);
}

// ------------------------------------------------------------------ early exit
// Left-to-right verification that reads only the rows up to each request's
// cut.  Round j is two launches: k_round streams the position-j rows of every
// request still undecided (and the residual row pairs of the requests cut at
// j - 1), then k_decide_round decides position j of those requests and lists
// the kept ones, their next rows and the new residual sweeps for round j + 1.
// Lists rotate over three buffers; k_round of round j clears the counts of
// the list that k_decide_round of round j fills.  No kernel waits on another
// wavefront: every hand-over is a kernel boundary.

// One workgroup: offsets as in k_plan, every output set to -1 (slots no round
// reaches keep it), round 0 lists every request with its position-0 rows.
__global__ __launch_bounds__(kPlanThreads) void k_plan_ee(Args a) {
  constexpr int kPlanWaves = kPlanThreads / kWave;
  __shared__ long long s_wk[kPlanWaves];
  __shared__ long long s_wr[kPlanWaves];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid >> 6;
  if (tid == 0) s_bad = 0;
  for (long long i = tid; i < (long long)a.K + a.B; i += kPlanThreads) a.out[i] = -1;
  for (long long i = tid; i < a.K; i += kPlanThreads) {
    if (a.p_out) a.p_out[i] = -1.f;
    if (a.q_out) a.q_out[i] = -1.f;
  }
  for (int i = tid; i < a.B; i += kPlanThreads) {
    a.acc_len[i] = -1;
    if (a.resid_out) a.resid_out[i] = -1.f;
  }
  __syncthreads();
  long long carry_k = 0, carry_r = 0;
  for (int base = 0; base < a.B; base += kPlanThreads) {
    const int b = base + tid;
    long long k = 0;
    int g = 1;
    if (b < a.B) {
      int kk = a.num_draft[b];
      if (kk < 0 || kk > a.K || kk > a.max_k) {
        s_bad = 1;
        kk = 0;
      }
      k = kk;
      g = a.force_greedy ? 1 : (a.gmask ? (a.gmask[b] != 0) : 0);
    }
    const bool pair = (b < a.B) && !g && k > 0;
    const long long nr = (b < a.B) ? (pair ? 2 : 1) : 0;   // rows read in round 0
    const long long ik = wave_incl_scan_ll(k, lane);
    const long long ir = wave_incl_scan_ll(nr, lane);
    if (lane == kWave - 1) {
      s_wk[wv] = ik;
      s_wr[wv] = ir;
    }
    __syncthreads();
    long long pk = 0, pr = 0, tot_k = 0, tot_r = 0;
    for (int q = 0; q < kPlanWaves; ++q) {
      if (q < wv) {
        pk += s_wk[q];
        pr += s_wr[q];
      }
      tot_k += s_wk[q];
      tot_r += s_wr[q];
    }
    const long long off = carry_k + pk + ik - k;
    const long long roff = carry_r + pr + ir - nr;
    if (b < a.B) {
      ReqInfo r;
      r.off = (int)off;
      r.k = (int)k;
      r.greedy = g;
      r.a = 0;
      r.kind = KIND_NONE;
      r.y = -1;
      r.trow = -1;
      r.drow = -1;
      r.Mp = r.Mq = 0.f;
      r.pad0 = r.pad1 = 0;
      r.Sp = r.Sq = 0.0;
      a.ws.req[b] = r;
      a.ws.alive[b] = b;
      const long long trow = off + b;
      if (roff < 2ll * a.B && trow < (long long)a.K + a.B)
        a.ws.rows_r[roff] = (uint32_t)trow | (g ? kGreedyBit : 0u);
      if (pair && roff + 1 < 2ll * a.B && off < a.K)
        a.ws.rows_r[roff + 1] = (uint32_t)off | kDraftBit;
    }
    carry_k += tot_k;
    carry_r += tot_r;
    __syncthreads();
  }
  if (tid == 0) {
    const bool bad = s_bad != 0 || carry_k != a.K;
    Header* h = a.ws.hdr;
    h->error = bad ? 1 : 0;
    h->n_resid = 0;
    h->n_rows3[0] = bad ? 0 : (int)carry_r;
    h->n_res3[0] = 0;
    h->n_alive3[0] = bad ? 0 : a.B;
    h->n_rows3[1] = 0;
    h->n_res3[1] = 0;
    h->n_alive3[1] = 0;
    h->n_rows = 0;
    h->n_units = 0;
  }
}

// Decision of position j of request b by one wavefront.  Lane 0 combines the
// target row and lane 1 the draft row with the per-row combines of k_decide,
// so both paths see the same statistics bit for bit.
template <class L>
__device__ __forceinline__ void decide_position(const Args& a, int b, int j, int nxt, int lane) {
  Header* hdr = a.ws.hdr;
  const ReqInfo R = a.ws.req[b];
  const int k = R.k;
  const bool g = R.greedy != 0;
  const int trow = R.off + b + j;
  const int drow = R.off + j;
  const int nseg = a.nseg;
  if (j == 0 && !g) {
    // a stochastic request with a draft token outside [0, V) reports -1
    // everywhere, as on the all-rows path: all its tokens are tested up front
    bool bad = false;
    for (int i = lane; i < k; i += kWave) {
      const int y = a.tokens[R.off + i];
      bad |= (y < 0 || y >= a.V);
    }
    if (__any(bad)) return;             // outputs keep the -1 written by the plan
  }
  // loads that depend only on the request are issued before the row combines
  int y = 0;
  float zy = 0.f, dy = 0.f, u = 0.f;
  if (lane == 0 && j < k) {
    y = a.tokens[drow];
    if (!g) {
      u = a.u_accept[drow];
      if (y >= 0 && y < a.V) {          // checked for every token in round 0
        zy = logit_at<L>(a.target, trow, a.tld, y);
        dy = logit_at<L>(a.draft, drow, a.dld, y);
      }
    }
  }
  const bool draft_row = !g && j < k;
  float M = 0.f;
  double S = 0.0;
  int amax = INT_MAX;
  if (lane == 0 && g) {
    row_argmax(a.ws.pt + (int64_t)trow * nseg, nseg, amax);
  } else if (lane == 0 || (lane == 1 && draft_row)) {
    const Partial* P = (lane == 0) ? a.ws.pt + (int64_t)trow * nseg
                                   : a.ws.pd + (int64_t)drow * nseg;
    row_softmax(P, nseg, a.c_hi, a.c_lo, M, S);
  }
  const float Mq = __shfl(M, 1);
  const double Sq = __shfl(S, 1);
  M = __shfl(M, 0);
  S = __shfl(S, 0);
  amax = __shfl(amax, 0);
  if (j == k) {                         // every draft kept: the final token
    if (g) {
      if (lane == 0) {
        a.acc_len[b] = k;
        a.out[trow] = (amax == INT_MAX) ? -1 : amax;
      }
    } else if (lane == 0) {             // drawn by k_finalize after the last round
      ReqInfo Wr = R;
      Wr.a = k;
      Wr.trow = trow;
      Wr.kind = KIND_BONUS;
      Wr.Mp = M;
      Wr.Sp = S;
      a.acc_len[b] = k;
      a.ws.req[b] = Wr;
    }
    return;
  }
  if (lane != 0) return;
  bool rej;
  if (g) {
    rej = (y != amax);
  } else {
    const double py = exp(((double)zy - (double)M) / a.T64) / S;
    const double qy = exp(((double)dy - (double)Mq) / a.T64) / Sq;
    rej = !((double)u * qy < py);
    if (a.p_out) a.p_out[drow] = (float)py;
    if (a.q_out) a.q_out[drow] = (float)qy;
  }
  if (!rej) {                           // keep y_j, list position j + 1
    a.out[trow] = y;
    const int ia = atomicAdd(&hdr->n_alive3[nxt], 1);
    a.ws.alive[(int64_t)nxt * a.B + ia] = b;
    const bool pair = !g && j + 1 < k;
    const int ir = atomicAdd(&hdr->n_rows3[nxt], pair ? 2 : 1);
    uint32_t* rows = a.ws.rows_r + (int64_t)nxt * 2 * a.B;
    rows[ir] = (uint32_t)(trow + 1) | (g ? kGreedyBit : 0u);
    if (pair) rows[ir + 1] = (uint32_t)(drow + 1) | kDraftBit;
  } else {                              // cut at j
    a.acc_len[b] = j;
    if (g) {
      a.out[trow] = (amax == INT_MAX) ? -1 : amax;
    } else {                            // pair swept in round j + 1, drawn by k_finalize
      ReqInfo Wr = R;
      Wr.a = j;
      Wr.trow = trow;
      Wr.drow = drow;
      Wr.y = y;
      Wr.kind = KIND_RESID;
      Wr.Mp = M;
      Wr.Sp = S;
      Wr.Mq = Mq;
      Wr.Sq = Sq;
      a.ws.req[b] = Wr;
      const int ir = atomicAdd(&hdr->n_res3[nxt], 1);
      a.ws.res_r[(int64_t)nxt * a.B + ir] = b;
    }
  }
}

// Round j (a.ee_round), streaming half: persistent grid over the round's
// units, row units first, then residual units.
template <class L>
__global__ __launch_bounds__(kBlock) void k_round(Args a) {
  using Elem = typename L::Elem;
  const int lane = threadIdx.x & (kWave - 1);
  const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int W = gridDim.x * kWavesPerBlock;
  const int j = a.ee_round;
  const int cur = j % 3, nxt = (j + 1) % 3;
  Header* hdr = a.ws.hdr;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    // the lists k_decide_round of this round fills; round j - 2 read them
    hdr->n_rows3[nxt] = 0;
    hdr->n_res3[nxt] = 0;
    hdr->n_alive3[nxt] = 0;
  }
  const int n_s = hdr->n_rows3[cur] * a.nseg;
  const int n_units = n_s + hdr->n_res3[cur] * a.nrseg;
  const uint32_t* rows = a.ws.rows_r + (int64_t)cur * 2 * a.B;
  const int* res = a.ws.res_r + (int64_t)cur * a.B;
  const Elem* tgt = static_cast<const Elem*>(a.target);
  const Elem* drf = static_cast<const Elem*>(a.draft);
  for (int u = gw; u < n_units; u += W) {
    if (u < n_s) {
      const int ri = u / a.nseg;
      const int seg = u - ri * a.nseg;
      const uint32_t desc = rows[ri];
      const int row = (int)(desc & kRowMask);
      const bool is_draft = (desc & kDraftBit) != 0;
      const int s0 = seg * a.seg;
      const int s1 = min(s0 + a.seg, a.V);
      const Elem* base = is_draft ? drf + (int64_t)row * a.dld : tgt + (int64_t)row * a.tld;
      Partial* out = (is_draft ? a.ws.pd : a.ws.pt) + (int64_t)row * a.nseg + seg;
      if (desc & kGreedyBit)
        argmax_unit<L, kRoundUnroll>(base, s0, s1, lane, out);
      else
        softmax_unit<L, kRoundUnroll>(base, s0, s1, lane, a, out);
    } else {                            // residual unit of a request cut at j - 1
      const int v = u - n_s;
      const int ri = v / a.nrseg;
      const int seg = v - ri * a.nrseg;
      const int b = res[ri];
      const ReqInfo R = a.ws.req[b];
      const Elem* tp = tgt + (int64_t)R.trow * a.tld;
      const Elem* dp = drf + (int64_t)R.drow * a.dld;
      const int s0 = seg * a.rseg;
      const int s1 = min(s0 + a.rseg, a.V);
      const double tot = resid_unit<L, kRoundUnroll>(tp, dp, resid_weights(R, a), R.y, s0, s1, lane);
      if (lane == 0) a.ws.rp[(int64_t)b * a.nrseg + seg] = tot;
    }
  }
}

// Round j, deciding half: one wavefront per request whose position-j rows the
// round streamed.
template <class L>
__global__ __launch_bounds__(kBlock) void k_decide_round(Args a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int W = gridDim.x * kWavesPerBlock;
  const int j = a.ee_round;
  const int cur = j % 3, nxt = (j + 1) % 3;
  const int nal = a.ws.hdr->n_alive3[cur];
  for (int w = gw; w < nal; w += W)
    decide_position<L>(a, a.ws.alive[(int64_t)cur * a.B + w], j, nxt, lane);
}

// ------------------------------------------------------------------ token trees
// Greedy verification of a token tree (chzhyang, "Speculative Decoding: ...",
// section 5 DDTree): from the root, follow the child whose token is the
// target's choice at the current node; when no child carries it, that choice
// is the bonus token.  Request b owns nodes off .. off + n_b - 1 (node 0 the
// root), and node i's target row is row off + i.  ReqInfo fields for trees:
// off, k = n_b, a = nodes accepted so far, trow = row of the current node.

// One workgroup: node offsets, every output -1, the row list (all rows) or
// the round-0 list of walking requests (early exit; every request at its root).
__global__ __launch_bounds__(kPlanThreads) void k_tree_plan(Args a) {
  constexpr int kPlanWaves = kPlanThreads / kWave;
  __shared__ long long s_wn[kPlanWaves];
  __shared__ int s_bad, s_na;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid >> 6;
  const bool rounds = a.ee_round >= 0;
  if (tid == 0) {
    s_bad = 0;
    s_na = 0;
  }
  for (long long i = tid; i < a.K; i += kPlanThreads) {
    a.out[i] = -1;
    a.path[i] = -1;
    if (!rounds) a.ws.rowdesc[i] = (uint32_t)i | kGreedyBit;
  }
  for (int i = tid; i < a.B; i += kPlanThreads) a.acc_len[i] = -1;
  __syncthreads();
  long long carry = 0;
  for (int base = 0; base < a.B; base += kPlanThreads) {
    const int b = base + tid;
    long long n = 0;
    if (b < a.B) {
      const int nn = a.num_draft[b];
      if (nn < 1 || nn > a.K) s_bad = 1;
      else n = nn;
    }
    const long long incl = wave_incl_scan_ll(n, lane);
    if (lane == kWave - 1) s_wn[wv] = incl;
    __syncthreads();
    long long pre = 0, tot = 0;
    for (int q = 0; q < kPlanWaves; ++q) {
      if (q < wv) pre += s_wn[q];
      tot += s_wn[q];
    }
    const long long off = carry + pre + incl - n;
    if (b < a.B) {
      ReqInfo r;
      r.off = (int)off;
      r.k = (int)n;
      r.greedy = 1;
      r.a = 0;
      r.kind = KIND_NONE;
      r.y = -1;
      r.trow = (int)off;
      r.drow = -1;
      r.Mp = r.Mq = 0.f;
      r.pad0 = r.pad1 = 0;
      r.Sp = r.Sq = 0.0;
      if (rounds && n >= 1) a.ws.alive[atomicAdd(&s_na, 1)] = b;   // round 0: at the root
      a.ws.req[b] = r;
    }
    carry += tot;
    __syncthreads();
  }
  if (tid == 0) {
    const bool bad = s_bad != 0 || carry != a.K;
    Header* h = a.ws.hdr;
    h->error = bad ? 1 : 0;
    h->n_rows = bad ? 0 : a.K;
    h->n_units = 0;
    h->n_resid = 0;
    h->n_alive3[0] = (rounds && !bad) ? s_na : 0;   // (list order is free)
    h->n_alive3[1] = 0;
  }
}

// 0 <= parent < node for every non-root node of the request (one wavefront).
__device__ bool tree_parents_ok(const Args& a, const ReqInfo& R, int lane) {
  bool bad = false;
  for (int i = 1 + lane; i < R.k; i += kWave) {
    const int p = a.parent[R.off + i];
    bad |= (p < 0 || p >= i);
  }
  return !__any(bad);
}

// Lexicographic (max, lowest id) over the unit partials P[0 .. nseg) of one
// row: lanes over units, then a wavefront reduction (exact in any order).
__device__ int wave_row_argmax(const Partial* P, int nseg, int lane) {
  float bm = -INFINITY;
  int bi = INT_MAX;
  for (int s = lane; s < nseg; s += kWave) {
    const Partial p = P[s];
    if (p.m > bm || (p.m == bm && p.idx < bi)) {
      bm = p.m;
      bi = p.idx;
    }
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) {
    const float ob = __shfl_xor(bm, o);
    const int oi = __shfl_xor(bi, o);
    if (ob > bm || (ob == bm && oi < bi)) {
      bm = ob;
      bi = oi;
    }
  }
  return bi;
}

// One step of the walk for request b at its current node (global row trow),
// whose unit partials are P: the target's choice, then the lowest-index child
// of the node carrying that token.  Lane 0 writes the path and token slots.
// Returns the child's local index, or -1 when the walk ends (acc_len written).
__device__ int tree_step(const Args& a, int b, const ReqInfo& R, const Partial* P, int t,
                         int lane) {
  const int cur = R.trow - R.off;
  const int choice = wave_row_argmax(P, a.nseg, lane);
  int follow = -1;
  if (choice != INT_MAX) {
    for (int i0 = cur + 1; i0 < R.k && follow < 0; i0 += kWave) {
      const int i = i0 + lane;
      const bool m = i < R.k && a.parent[R.off + i] == cur && a.tokens[R.off + i] == choice;
      const unsigned long long hit = __ballot(m);
      if (hit) follow = i0 + __ffsll((long long)hit) - 1;
    }
  }
  if (lane == 0) {
    a.path[R.off + t] = cur;
    a.out[R.off + t] = (choice == INT_MAX) ? -1 : choice;
    if (follow < 0) a.acc_len[b] = t;
  }
  return follow;
}

// All-rows walk: one wavefront per request after k_stats has summarised every
// node row.
__global__ __launch_bounds__(kBlock) void k_tree_walk(Args a) {
  if (a.ws.hdr->error) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int W = gridDim.x * kWavesPerBlock;
  for (int b = gw; b < a.B; b += W) {
    ReqInfo R = a.ws.req[b];
    if (!tree_parents_ok(a, R, lane)) continue;   // outputs keep -1
    for (int t = 0;; ++t) {             // every step moves to a higher node index
      const int f = tree_step(a, b, R, a.ws.pt + (int64_t)R.trow * a.nseg, t, lane);
      if (f < 0) break;
      R.trow = R.off + f;
    }
  }
}

// Early-exit rounds: round j streams the row of the current node of every
// request still walking (argmax units of kTreeSegBytes, partials kept per
// request: a round reads at most B rows, so small units keep every CU busy),
// then one wavefront per such request takes one step.  Lists of walking
// requests rotate over three buffers.
template <class L>
__global__ __launch_bounds__(kBlock) void k_tree_round(Args a) {
  using Elem = typename L::Elem;
  const int lane = threadIdx.x & (kWave - 1);
  const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int W = gridDim.x * kWavesPerBlock;
  const int j = a.ee_round;
  const int cur = j % 3, nxt = (j + 1) % 3;
  Header* hdr = a.ws.hdr;
  if (blockIdx.x == 0 && threadIdx.x == 0) hdr->n_alive3[nxt] = 0;
  const int n_units = hdr->n_alive3[cur] * a.nseg;
  const int* alive = a.ws.alive + (int64_t)cur * a.B;
  const Elem* tgt = static_cast<const Elem*>(a.target);
  for (int u = gw; u < n_units; u += W) {
    const int w = u / a.nseg;
    const int seg = u - w * a.nseg;
    const int b = alive[w];
    const int row = a.ws.req[b].trow;
    const int s0 = seg * a.seg;
    const int s1 = min(s0 + a.seg, a.V);
    argmax_unit<L>(tgt + (int64_t)row * a.tld, s0, s1, lane,
                   a.ws.pt + (int64_t)b * a.nseg + seg);
  }
}

__global__ __launch_bounds__(kBlock) void k_tree_step_round(Args a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int W = gridDim.x * kWavesPerBlock;
  const int j = a.ee_round;
  const int cur = j % 3, nxt = (j + 1) % 3;
  Header* hdr = a.ws.hdr;
  const int nal = hdr->n_alive3[cur];
  for (int w = gw; w < nal; w += W) {
    const int b = a.ws.alive[(int64_t)cur * a.B + w];
    ReqInfo R = a.ws.req[b];
    if (j == 0 && !tree_parents_ok(a, R, lane)) continue;   // outputs keep -1
    const int f = tree_step(a, b, R, a.ws.pt + (int64_t)b * a.nseg, j, lane);
    if (f < 0) continue;
    if (j == a.max_k) {
      // the walk would accept more than max_depth nodes: an input error, the
      // request reports -1 everywhere
      for (int i = lane; i <= j; i += kWave) {
        a.path[R.off + i] = -1;
        a.out[R.off + i] = -1;
      }
      continue;
    }
    if (lane == 0) {
      a.ws.req[b].trow = R.off + f;
      const int ia = atomicAdd(&hdr->n_alive3[nxt], 1);
      a.ws.alive[(int64_t)nxt * a.B + ia] = b;
    }
  }
}

// ------------------------------------------------------------------ adaptive length
// Confidence-driven verification length (chzhyang, "Speculative Decoding: ...",
// section 5 DSpark; section 2 for time per token): request b keeps the prefix
// length k in 0..N maximising (1 + s_1 + ... + s_k) / cost[k], s_j = c_1 ... c_j,
// ties to the smallest k, then the kept windows are packed back to back.  The
// arithmetic is fp64 in a fixed order: s = s * c, total = total + s, ratio =
// total / cost[k].
struct AdaptArgs {
  int B, N;
  const float* conf;
  const double* cost;
  const int* tokens;
  int* num_draft;
  int* offsets;
  int* tokens_out;
  int* src_index;
  double* progress;
};

__global__ __launch_bounds__(kPlanThreads) void k_adaptive(AdaptArgs a) {
  constexpr int kPlanWaves = kPlanThreads / kWave;
  __shared__ long long s_w[kPlanWaves];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid >> 6;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  for (int k = tid; k <= a.N; k += kPlanThreads) {
    // positive and finite, tested on the bits (device code assumes no NaNs)
    const unsigned long long u = (unsigned long long)__double_as_longlong(a.cost[k]);
    const bool ok = (u >> 63) == 0 && u != 0 && ((u >> 52) & 0x7ffull) != 0x7ffull;
    if (!ok) s_bad = 1;
  }
  __syncthreads();
  const bool bad = s_bad != 0;
  long long carry = 0;
  for (int base = 0; base < a.B; base += kPlanThreads) {
    const int b = base + tid;
    int kb = 0;
    double prog = 1.0;
    if (b < a.B && !bad) {
      const float* c = a.conf + (int64_t)b * a.N;
      double s = 1.0, total = 1.0;
      double best = 1.0 / a.cost[0];
      for (int j = 0; j < a.N; ++j) {
        s = s * (double)c[j];
        total = total + s;
        const double r = total / a.cost[j + 1];
        if (r > best) {
          best = r;
          kb = j + 1;
          prog = total;
        }
      }
    }
    const long long incl = wave_incl_scan_ll(kb, lane);
    if (lane == kWave - 1) s_w[wv] = incl;
    __syncthreads();
    long long pre = 0, tot = 0;
    for (int q = 0; q < kPlanWaves; ++q) {
      if (q < wv) pre += s_w[q];
      tot += s_w[q];
    }
    const long long off = carry + pre + incl - kb;
    if (b < a.B) {
      a.num_draft[b] = bad ? -1 : kb;
      a.offsets[b] = (int)off;
      if (a.progress) a.progress[b] = bad ? -1.0 : prog;
      for (int i = 0; i < kb; ++i) {
        const int src = b * a.N + i;
        a.tokens_out[off + i] = a.tokens[src];
        if (a.src_index) a.src_index[off + i] = src;
      }
    }
    carry += tot;
    __syncthreads();
  }
  if (tid == 0) a.offsets[a.B] = (int)carry;
}

// dst row r = src row index[r] for r < min(*count, max_rows); rows whose index
// lies outside [0, src_rows) are left unwritten.  Persistent grid over 32 KiB
// pieces of the destination rows; nontemporal 16-byte loads and stores when
// both layouts allow them.
struct GatherArgs {
  int V, max_rows, src_rows, es, vec;
  int64_t src_ld, dst_ld;
  const uint8_t* src;
  uint8_t* dst;
  const int* index;
  const int* count;
};

__global__ __launch_bounds__(kBlock) void k_gather_rows(GatherArgs g) {
  const int gt = blockIdx.x * kBlock + threadIdx.x;
  const int nthreads = gridDim.x * kBlock;
  const int rows = min(*g.count, g.max_rows);
  const long long row_bytes = (long long)g.V * g.es;
  constexpr int kPiece = 32768;
  const long long pieces = (row_bytes + kPiece - 1) / kPiece;
  const long long n_units = (long long)max(rows, 0) * pieces;
  const int gw = gt >> 6;
  const int lane = threadIdx.x & (kWave - 1);
  const int W = nthreads >> 6;
  for (long long u = gw; u < n_units; u += W) {
    const int r = (int)(u / pieces);
    const long long p0 = (u - (long long)r * pieces) * kPiece;
    const long long p1 = min(p0 + kPiece, row_bytes);
    const int sr = g.index[r];
    if (sr < 0 || sr >= g.src_rows) continue;
    const uint8_t* s = g.src + (int64_t)sr * g.src_ld * g.es;
    uint8_t* d = g.dst + (int64_t)r * g.dst_ld * g.es;
    if (g.vec) {
      long long o = p0 + (long long)lane * 16;
      for (; o + 16 <= p1; o += kWave * 16) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(s + o));
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(d + o));
      }
      for (long long t = o; t < p1; t += g.es) {   // row tail shorter than 16 bytes
        if (g.es == 4) *reinterpret_cast<uint32_t*>(d + t) = *reinterpret_cast<const uint32_t*>(s + t);
        else *reinterpret_cast<uint16_t*>(d + t) = *reinterpret_cast<const uint16_t*>(s + t);
      }
    } else {
      for (long long o = p0 + (long long)lane * g.es; o < p1; o += kWave * g.es) {
        if (g.es == 4) *reinterpret_cast<uint32_t*>(d + o) = *reinterpret_cast<const uint32_t*>(s + o);
        else *reinterpret_cast<uint16_t*>(d + o) = *reinterpret_cast<const uint16_t*>(s + o);
      }
    }
  }
}

// ------------------------------------------------------------------ acceptance statistics
// One workgroup: LDS histograms of accepted and proposed lengths over
// [0, max_pos] (larger values fold into the top bin, which keeps every
// #{x >= j} for j <= max_pos exact), 64-bit totals, suffix sums, fp64 ratios.
constexpr int kStatsThreads = 1024;
constexpr int kMaxStatsPos = 4096;

__global__ __launch_bounds__(kStatsThreads) void k_accept_stats(const int* acc, const int* nd,
                                                               int B, int max_pos, double* out) {
  extern __shared__ unsigned int s_hist[];          // [2 * (max_pos + 1)]
  __shared__ unsigned long long s_sa, s_sk, s_n;
  unsigned int* h_a = s_hist;
  unsigned int* h_k = s_hist + (max_pos + 1);
  for (int i = threadIdx.x; i < 2 * (max_pos + 1); i += kStatsThreads) s_hist[i] = 0u;
  if (threadIdx.x == 0) {
    s_sa = 0ull;
    s_sk = 0ull;
    s_n = 0ull;
  }
  __syncthreads();
  long long sa = 0, sk = 0, n = 0;
  for (int b = threadIdx.x; b < B; b += kStatsThreads) {
    const int a = acc[b];
    if (a < 0) continue;
    const int k = nd[b];
    atomicAdd(&h_a[min(a, max_pos)], 1u);
    atomicAdd(&h_k[min(max(k, 0), max_pos)], 1u);
    sa += a;
    sk += k;
    n += 1;
  }
  atomicAdd(&s_sa, (unsigned long long)sa);
  atomicAdd(&s_sk, (unsigned long long)sk);
  atomicAdd(&s_n, (unsigned long long)n);
  __syncthreads();
  if (threadIdx.x == 0) {
    const long long tn = (long long)s_n, ta = (long long)s_sa, tk = (long long)s_sk;
    const double mean = tn ? (double)ta / (double)tn : -1.0;
    out[0] = (double)tn;
    out[1] = mean;
    out[2] = tn ? 1.0 + mean : -1.0;
    out[3] = tk ? (double)ta / (double)tk : -1.0;
    unsigned long long ca = 0ull, ck = 0ull;
    for (int j = max_pos; j >= 1; --j) {
      ca += h_a[j];
      ck += h_k[j];
      out[3 + j] = ck ? (double)ca / (double)ck : -1.0;
    }
  }
}

// ------------------------------------------------------------------ host helpers
size_t align_up(size_t x, size_t al) { return (x + al - 1) / al * al; }

struct Sizes {
  size_t off_hdr, off_req, off_rowdesc, off_resid, off_pt, off_pd, off_rp, off_rows_r, off_res_r,
      off_alive, total;
};

bool compute_sizes(long long B, long long K, long long V, Sizes* z) {
  if (B < 1 || K < 0 || V < 1 || V > (1ll << 30)) return false;
  if (K + B >= (1ll << 29)) return false;
  const long long nseg = (V + kSegMinElems - 1) / kSegMinElems;
  const long long nrseg = (V + kRSegMinElems - 1) / kRSegMinElems;
  // unit counts are 32-bit in the kernels; an early-exit round can list row
  // units and residual units together
  if ((2 * K + B) * nseg + B * nrseg >= (1ll << 31)) return false;
  size_t o = 0;
  z->off_hdr = o; o = align_up(o + sizeof(Header), 256);
  z->off_req = o; o = align_up(o + sizeof(ReqInfo) * (size_t)B, 256);
  z->off_rowdesc = o; o = align_up(o + 4 * (size_t)(2 * K + B), 256);
  z->off_resid = o; o = align_up(o + 4 * (size_t)B, 256);
  z->off_pt = o; o = align_up(o + sizeof(Partial) * (size_t)((K + B) * nseg), 256);
  z->off_pd = o; o = align_up(o + sizeof(Partial) * (size_t)(K * nseg), 256);
  z->off_rp = o; o = align_up(o + sizeof(double) * (size_t)(B * nrseg), 256);
  z->off_rows_r = o; o = align_up(o + 4 * (size_t)(6 * B), 256);
  z->off_res_r = o; o = align_up(o + 4 * (size_t)(3 * B), 256);
  z->off_alive = o; o = align_up(o + 4 * (size_t)(3 * B), 256);
  z->total = o + 256;   // slack for aligning the caller's pointer
  return true;
}

thread_local void* g_ev_begin = nullptr;
thread_local void* g_ev_end = nullptr;
thread_local int g_launch_plan = 0;   // 0 automatic, 1 multi-kernel, 2 single launch

// Logit bytes up to which a batch runs as one launch (one workgroup per
// request): below this the five-kernel path is bound by launch latency.
constexpr long long kFusedMaxBytes = 48ll << 20;
constexpr int kFusedMaxRequests = 2048;

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

void split_constant(double T, float* hi, float* lo, double* c64) {
  const double c = 1.4426950408889634 / T;   // log2(e) / T
  float h = (float)c;
  if ((double)h > c) h = nextafterf(h, 0.f);  // round toward zero so that c_lo >= 0
  float l = (float)(c - (double)h);
  if (!(l >= 1e-30f)) l = 1e-30f;             // keep c_lo > 0: -inf * c_lo stays -inf
  *hi = h;
  *lo = l;
  *c64 = c;
}

// Resident workgroups per CU for a kernel, from the occupancy calculator
// (cached per device); the persistent grids are sized to exactly fill the chip.
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

template <class L>
void launch_fused(const Args& a, hipStream_t st) {
  if (g_ev_begin && g_ev_end) (void)hipEventRecord((hipEvent_t)g_ev_begin, st);
  k_fused<L><<<a.B, kFusedThreads, 0, st>>>(a);
  if (g_ev_begin && g_ev_end) (void)hipEventRecord((hipEvent_t)g_ev_end, st);
}

template <class L>
void launch_all(const Args& a, hipStream_t st, int dev, bool sample) {
  static std::atomic<int> occ_stats[64];
  static std::atomic<int> occ_resid[64];
  const long long cus = cu_count(dev);
  const long long units_stats = (2ll * a.K + a.B) * a.nseg;
  const long long units_resid = (long long)a.B * a.nrseg;
  const long long cap_s = cus * resident_blocks(occ_stats, k_stats<L>, dev);
  const int grid_stats = (int)std::max(1ll, std::min(cap_s, (units_stats + kWavesPerBlock - 1) / kWavesPerBlock));
  k_plan<<<1, kPlanThreads, 0, st>>>(a);
  if (g_ev_begin && g_ev_end) (void)hipEventRecord((hipEvent_t)g_ev_begin, st);
  k_stats<L><<<grid_stats, kBlock, 0, st>>>(a);
  if (g_ev_begin && g_ev_end) (void)hipEventRecord((hipEvent_t)g_ev_end, st);
  k_decide<L><<<(a.B + kWavesPerBlock - 1) / kWavesPerBlock, kBlock, 0, st>>>(a);
  if (sample) {
    const long long cap_r = cus * resident_blocks(occ_resid, k_resid<L>, dev);
    const int grid_resid = (int)std::max(1ll, std::min(cap_r, (units_resid + kWavesPerBlock - 1) / kWavesPerBlock));
    k_resid<L><<<grid_resid, kBlock, 0, st>>>(a);
    k_finalize<L><<<a.B, kBlock, 0, st>>>(a);
  }
}

template <class L>
void launch_early_exit(const Args& a, hipStream_t st, int dev, bool sample) {
  static std::atomic<int> occ_round[64];
  const long long cus = cu_count(dev);
  const long long units_max = 2ll * a.B * a.nseg + (long long)a.B * a.nrseg;
  const long long cap = cus * resident_blocks(occ_round, k_round<L>, dev);
  const int grid = (int)std::max(1ll, std::min(cap, (units_max + kWavesPerBlock - 1) / kWavesPerBlock));
  const int grid_dec = (int)std::max(1ll, std::min(cus * kBlocksPerCU, ((long long)a.B + kWavesPerBlock - 1) / kWavesPerBlock));
  k_plan_ee<<<1, kPlanThreads, 0, st>>>(a);
  if (g_ev_begin && g_ev_end) (void)hipEventRecord((hipEvent_t)g_ev_begin, st);
  for (int j = 0; j <= a.max_k; ++j) {
    Args r = a;
    r.ee_round = j;
    k_round<L><<<grid, kBlock, 0, st>>>(r);
    k_decide_round<L><<<grid_dec, kBlock, 0, st>>>(r);
  }
  if (g_ev_begin && g_ev_end) (void)hipEventRecord((hipEvent_t)g_ev_end, st);
  if (sample) k_finalize<L><<<a.B, kBlock, 0, st>>>(a);
}

int32_t run(const sv_batch_t* bt, bool sample, float temperature, const uint8_t* gmask,
            const float* u_accept, const float* u_final, int32_t* acc_len, int32_t* out,
            float* p_out, float* q_out, float* resid_out, void* ws, size_t ws_bytes,
            void* stream, bool early_exit, int max_k) {
  // ---- host-side checks: nothing below touches the GPU until they pass
  if (!bt) return SV_ERR_INVALID_ARG;
  if (early_exit && (max_k < 0 || max_k > kMaxEarlyExitRounds)) return SV_ERR_INVALID_ARG;
  const long long B = bt->B, K = bt->K, V = bt->V;
  Sizes z;
  if (!compute_sizes(B, K, V, &z)) return SV_ERR_INVALID_ARG;
  if (bt->dtype != SV_F32 && bt->dtype != SV_BF16) return SV_ERR_UNSUPPORTED;
  const int es = bt->dtype == SV_F32 ? 4 : 2;
  if (!bt->num_draft || !bt->target || !acc_len || !out) return SV_ERR_INVALID_ARG;
  if (K > 0 && !bt->draft_tokens) return SV_ERR_INVALID_ARG;
  if (bt->target_ld < V || bt->target_ld > (1ll << 40)) return SV_ERR_INVALID_ARG;
  if ((uintptr_t)bt->target % es != 0) return SV_ERR_INVALID_ARG;
  const bool need_draft = sample && K > 0;
  if (sample) {
    if (!u_final) return SV_ERR_INVALID_ARG;
    if (!(temperature > 0.f) || !isfinite(temperature)) return SV_ERR_INVALID_ARG;
    if (K > 0 && (!u_accept || !bt->draft)) return SV_ERR_INVALID_ARG;
  }
  if (need_draft) {
    if (bt->draft_ld < V || bt->draft_ld > (1ll << 40)) return SV_ERR_INVALID_ARG;
    if ((uintptr_t)bt->draft % es != 0) return SV_ERR_INVALID_ARG;
  }
  if (!ws) return SV_ERR_WORKSPACE;
  if (ws_bytes < z.total) return SV_ERR_WORKSPACE;

  // ---- argument block
  const uintptr_t wb = align_up((uintptr_t)ws, 256);
  Args a;
  a.B = (int)B;
  a.K = (int)K;
  a.V = (int)V;
  a.seg = kSegBytes / es;
  a.nseg = (int)((V + a.seg - 1) / a.seg);
  a.rseg = kRSegBytes / es;
  a.nrseg = (int)((V + a.rseg - 1) / a.rseg);
  a.force_greedy = sample ? 0 : 1;
  a.tld = bt->target_ld;
  a.dld = need_draft ? bt->draft_ld : 0;
  a.target = bt->target;
  a.draft = need_draft ? bt->draft : nullptr;
  a.num_draft = bt->num_draft;
  a.tokens = bt->draft_tokens;
  a.gmask = sample ? gmask : nullptr;
  a.u_accept = u_accept;
  a.u_final = u_final;
  a.acc_len = acc_len;
  a.out = out;
  a.p_out = sample ? p_out : nullptr;
  a.q_out = sample ? q_out : nullptr;
  a.resid_out = sample ? resid_out : nullptr;
  if (sample) {
    a.T64 = (double)temperature;
    split_constant(a.T64, &a.c_hi, &a.c_lo, &a.c64);
  } else {
    a.T64 = 1.0;
    split_constant(1.0, &a.c_hi, &a.c_lo, &a.c64);
  }
  a.ws.hdr = reinterpret_cast<Header*>(wb + z.off_hdr);
  a.ws.req = reinterpret_cast<ReqInfo*>(wb + z.off_req);
  a.ws.rowdesc = reinterpret_cast<uint32_t*>(wb + z.off_rowdesc);
  a.ws.resid_list = reinterpret_cast<int*>(wb + z.off_resid);
  a.ws.pt = reinterpret_cast<Partial*>(wb + z.off_pt);
  a.ws.pd = reinterpret_cast<Partial*>(wb + z.off_pd);
  a.ws.rp = reinterpret_cast<double*>(wb + z.off_rp);
  a.ws.rows_r = reinterpret_cast<uint32_t*>(wb + z.off_rows_r);
  a.ws.res_r = reinterpret_cast<int*>(wb + z.off_res_r);
  a.ws.alive = reinterpret_cast<int*>(wb + z.off_alive);
  a.rowlist = a.ws.rowdesc;
  a.rowcount = &a.ws.hdr->n_rows;
  a.ee_round = -1;
  a.max_k = max_k;

  bool vec = ((uintptr_t)bt->target % 16 == 0) && ((bt->target_ld * es) % 16 == 0);
  if (need_draft) vec = vec && ((uintptr_t)bt->draft % 16 == 0) && ((bt->draft_ld * es) % 16 == 0);

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SV_ERR_HIP;
  hipStream_t st = static_cast<hipStream_t>(stream);

  (void)hipGetLastError();   // clear a stale error from earlier unrelated calls
  if (early_exit) {
    if (bt->dtype == SV_F32) {
      if (vec) launch_early_exit<F32>(a, st, dev, sample);
      else launch_early_exit<Scalar<F32>>(a, st, dev, sample);
    } else {
      if (vec) launch_early_exit<BF16>(a, st, dev, sample);
      else launch_early_exit<Scalar<BF16>>(a, st, dev, sample);
    }
  } else {
    // one launch for small batches (bytes bounded by all target rows plus a
    // draft row per drafted token)
    const long long bytes = (2 * K + B) * V * es;
    const bool fused = g_launch_plan == 2 ||
                       (g_launch_plan == 0 && bytes <= kFusedMaxBytes && B <= kFusedMaxRequests);
    if (bt->dtype == SV_F32) {
      if (fused) vec ? launch_fused<F32>(a, st) : launch_fused<Scalar<F32>>(a, st);
      else if (vec) launch_all<F32>(a, st, dev, sample);
      else launch_all<Scalar<F32>>(a, st, dev, sample);
    } else {
      if (fused) vec ? launch_fused<BF16>(a, st) : launch_fused<Scalar<BF16>>(a, st);
      else if (vec) launch_all<BF16>(a, st, dev, sample);
      else launch_all<Scalar<BF16>>(a, st, dev, sample);
    }
  }
  if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
  return SV_OK;
}


// ------------------------------------------------------------------ token trees (host)
struct TreeSizes {
  size_t off_hdr, off_req, off_rowdesc, off_pt, off_alive, total;
};

bool compute_tree_sizes(long long B, long long N, long long V, TreeSizes* z) {
  if (B < 1 || N < B || V < 1 || V > (1ll << 30)) return false;
  if (N >= (1ll << 29)) return false;
  const long long nseg = (V + kSegMinElems - 1) / kSegMinElems;
  const long long ntseg = (V + kTreeSegBytes / 4 - 1) / (kTreeSegBytes / 4);
  if (N * nseg >= (1ll << 31) || B * ntseg >= (1ll << 31)) return false;
  const long long npart = std::max(N * nseg, B * ntseg);   // all rows, or per-request rounds
  size_t o = 0;
  z->off_hdr = o; o = align_up(o + sizeof(Header), 256);
  z->off_req = o; o = align_up(o + sizeof(ReqInfo) * (size_t)B, 256);
  z->off_rowdesc = o; o = align_up(o + 4 * (size_t)N, 256);
  z->off_pt = o; o = align_up(o + sizeof(Partial) * (size_t)npart, 256);
  z->off_alive = o; o = align_up(o + 4 * (size_t)(3 * B), 256);
  z->total = o + 256;
  return true;
}

template <class L>
void launch_tree(const Args& a, hipStream_t st, int dev, bool early_exit) {
  static std::atomic<int> occ_stats[64];
  static std::atomic<int> occ_round[64];
  const long long cus = cu_count(dev);
  const int grid_walk = (int)std::max(1ll, std::min(cus * kBlocksPerCU, ((long long)a.B + kWavesPerBlock - 1) / kWavesPerBlock));
  k_tree_plan<<<1, kPlanThreads, 0, st>>>(a);
  if (!early_exit) {
    const long long units = (long long)a.K * a.nseg;
    const long long cap = cus * resident_blocks(occ_stats, k_stats<L>, dev);
    const int grid = (int)std::max(1ll, std::min(cap, (units + kWavesPerBlock - 1) / kWavesPerBlock));
    if (g_ev_begin && g_ev_end) (void)hipEventRecord((hipEvent_t)g_ev_begin, st);
    k_stats<L><<<grid, kBlock, 0, st>>>(a);
    if (g_ev_begin && g_ev_end) (void)hipEventRecord((hipEvent_t)g_ev_end, st);
    k_tree_walk<<<grid_walk, kBlock, 0, st>>>(a);
    return;
  }
  const long long units = (long long)a.B * a.nseg;
  const long long cap = cus * resident_blocks(occ_round, k_tree_round<L>, dev);
  const int grid = (int)std::max(1ll, std::min(cap, (units + kWavesPerBlock - 1) / kWavesPerBlock));
  if (g_ev_begin && g_ev_end) (void)hipEventRecord((hipEvent_t)g_ev_begin, st);
  for (int j = 0; j <= a.max_k; ++j) {
    Args r = a;
    r.ee_round = j;
    k_tree_round<L><<<grid, kBlock, 0, st>>>(r);
    k_tree_step_round<<<grid_walk, kBlock, 0, st>>>(r);
  }
  if (g_ev_begin && g_ev_end) (void)hipEventRecord((hipEvent_t)g_ev_end, st);
}

int32_t run_tree(const sv_tree_t* tr, int32_t* acc_len, int32_t* path, int32_t* out, void* ws,
                 size_t ws_bytes, void* stream, bool early_exit, int max_depth) {
  if (!tr) return SV_ERR_INVALID_ARG;
  if (early_exit && (max_depth < 0 || max_depth > kMaxEarlyExitRounds)) return SV_ERR_INVALID_ARG;
  const long long B = tr->B, N = tr->N, V = tr->V;
  TreeSizes z;
  if (!compute_tree_sizes(B, N, V, &z)) return SV_ERR_INVALID_ARG;
  if (tr->dtype != SV_F32 && tr->dtype != SV_BF16) return SV_ERR_UNSUPPORTED;
  const int es = tr->dtype == SV_F32 ? 4 : 2;
  if (!tr->num_nodes || !tr->parent || !tr->tokens || !tr->target) return SV_ERR_INVALID_ARG;
  if (!acc_len || !path || !out) return SV_ERR_INVALID_ARG;
  if (tr->target_ld < V || tr->target_ld > (1ll << 40)) return SV_ERR_INVALID_ARG;
  if ((uintptr_t)tr->target % es != 0) return SV_ERR_INVALID_ARG;
  if (!ws) return SV_ERR_WORKSPACE;
  if (ws_bytes < z.total) return SV_ERR_WORKSPACE;

  const uintptr_t wb = align_up((uintptr_t)ws, 256);
  Args a = {};
  a.B = (int)B;
  a.K = (int)N;
  a.V = (int)V;
  a.seg = (early_exit ? kTreeSegBytes : kSegBytes) / es;
  a.nseg = (int)((V + a.seg - 1) / a.seg);
  a.rseg = kRSegBytes / es;
  a.nrseg = (int)((V + a.rseg - 1) / a.rseg);
  a.force_greedy = 1;
  a.tld = tr->target_ld;
  a.target = tr->target;
  a.num_draft = tr->num_nodes;
  a.tokens = tr->tokens;
  a.parent = tr->parent;
  a.acc_len = acc_len;
  a.out = out;
  a.path = path;
  a.T64 = 1.0;
  split_constant(1.0, &a.c_hi, &a.c_lo, &a.c64);
  a.ws.hdr = reinterpret_cast<Header*>(wb + z.off_hdr);
  a.ws.req = reinterpret_cast<ReqInfo*>(wb + z.off_req);
  a.ws.rowdesc = reinterpret_cast<uint32_t*>(wb + z.off_rowdesc);
  a.ws.pt = reinterpret_cast<Partial*>(wb + z.off_pt);
  a.ws.alive = reinterpret_cast<int*>(wb + z.off_alive);
  a.rowlist = a.ws.rowdesc;
  a.rowcount = &a.ws.hdr->n_rows;
  a.ee_round = early_exit ? 0 : -1;
  a.max_k = early_exit ? max_depth : 0;

  const bool vec = ((uintptr_t)tr->target % 16 == 0) && ((tr->target_ld * es) % 16 == 0);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SV_ERR_HIP;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (tr->dtype == SV_F32) {
    if (vec) launch_tree<F32>(a, st, dev, early_exit);
    else launch_tree<Scalar<F32>>(a, st, dev, early_exit);
  } else {
    if (vec) launch_tree<BF16>(a, st, dev, early_exit);
    else launch_tree<Scalar<BF16>>(a, st, dev, early_exit);
  }
  if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
  return SV_OK;
}

}  // namespace

extern "C" size_t spec_verify_workspace_bytes(int32_t B, int32_t K, int32_t V) {
  Sizes z;
  if (!compute_sizes(B, K, V, &z)) return 0;
  return z.total;
}

extern "C" const char* spec_verify_status_string(int32_t status) {
  switch (status) {
    case SV_OK: return "ok";
    case SV_ERR_INVALID_ARG: return "invalid argument";
    case SV_ERR_UNSUPPORTED: return "unsupported dtype or dtype combination";
    case SV_ERR_WORKSPACE: return "workspace missing or too small";
    case SV_ERR_HIP: return "HIP runtime or kernel launch error";
    default: return "unknown status";
  }
}

extern "C" int32_t spec_verify_greedy(const sv_batch_t* batch, int32_t* accepted_len,
                                      int32_t* out_tokens, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  return run(batch, false, 1.f, nullptr, nullptr, nullptr, accepted_len, out_tokens, nullptr,
             nullptr, nullptr, workspace, workspace_bytes, stream, false, 0);
}

extern "C" int32_t spec_verify_greedy_early_exit(const sv_batch_t* batch, int32_t max_k,
                                                 int32_t* accepted_len, int32_t* out_tokens,
                                                 void* workspace, size_t workspace_bytes,
                                                 void* stream) {
  return run(batch, false, 1.f, nullptr, nullptr, nullptr, accepted_len, out_tokens, nullptr,
             nullptr, nullptr, workspace, workspace_bytes, stream, true, max_k);
}

extern "C" int32_t spec_verify_sample(const sv_batch_t* batch, float temperature,
                                      const uint8_t* greedy_mask, const float* u_accept,
                                      const float* u_final, int32_t* accepted_len,
                                      int32_t* out_tokens, float* p_draft, float* q_draft,
                                      float* resid_mass, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  return run(batch, true, temperature, greedy_mask, u_accept, u_final, accepted_len, out_tokens,
             p_draft, q_draft, resid_mass, workspace, workspace_bytes, stream, false, 0);
}

extern "C" int32_t spec_verify_sample_early_exit(const sv_batch_t* batch, int32_t max_k,
                                                 float temperature, const uint8_t* greedy_mask,
                                                 const float* u_accept, const float* u_final,
                                                 int32_t* accepted_len, int32_t* out_tokens,
                                                 float* p_draft, float* q_draft, float* resid_mass,
                                                 void* workspace, size_t workspace_bytes,
                                                 void* stream) {
  return run(batch, true, temperature, greedy_mask, u_accept, u_final, accepted_len, out_tokens,
             p_draft, q_draft, resid_mass, workspace, workspace_bytes, stream, true, max_k);
}

extern "C" int32_t spec_verify_accept_stats(const int32_t* accepted_len, const int32_t* num_draft,
                                            int32_t B, int32_t max_pos, double* out,
                                            void* stream) {
  if (!accepted_len || !num_draft || !out) return SV_ERR_INVALID_ARG;
  if (B < 1 || max_pos < 1 || max_pos > kMaxStatsPos) return SV_ERR_INVALID_ARG;
  (void)hipGetLastError();
  const size_t lds = sizeof(unsigned int) * 2 * (size_t)(max_pos + 1);
  k_accept_stats<<<1, kStatsThreads, lds, static_cast<hipStream_t>(stream)>>>(
      accepted_len, num_draft, B, max_pos, out);
  if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
  return SV_OK;
}

extern "C" int32_t spec_verify_set_launch_plan(int32_t plan) {
  if (plan < 0 || plan > 2) return SV_ERR_INVALID_ARG;
  g_launch_plan = plan;
  return SV_OK;
}

extern "C" int32_t spec_verify_set_profile_events(void* ev_begin, void* ev_end) {
  g_ev_begin = ev_begin;
  g_ev_end = ev_end;
  return SV_OK;
}

extern "C" size_t spec_verify_tree_workspace_bytes(int32_t B, int32_t N, int32_t V) {
  TreeSizes z;
  return compute_tree_sizes(B, N, V, &z) ? z.total : 0;
}

extern "C" int32_t spec_verify_tree_greedy(const sv_tree_t* tree, int32_t* accepted_len,
                                           int32_t* path_nodes, int32_t* out_tokens,
                                           void* workspace, size_t workspace_bytes, void* stream) {
  return run_tree(tree, accepted_len, path_nodes, out_tokens, workspace, workspace_bytes, stream,
                  false, 0);
}

extern "C" int32_t spec_verify_tree_greedy_early_exit(const sv_tree_t* tree, int32_t max_depth,
                                                      int32_t* accepted_len, int32_t* path_nodes,
                                                      int32_t* out_tokens, void* workspace,
                                                      size_t workspace_bytes, void* stream) {
  return run_tree(tree, accepted_len, path_nodes, out_tokens, workspace, workspace_bytes, stream,
                  true, max_depth);
}

extern "C" int32_t spec_verify_adaptive_length(int32_t B, int32_t N, const float* conf,
                                               const double* cost, const int32_t* draft_tokens,
                                               int32_t* num_draft, int32_t* offsets,
                                               int32_t* tokens_out, int32_t* src_index,
                                               double* progress, void* stream) {
  if (B < 1 || N < 0 || N > kMaxEarlyExitRounds || (long long)B * (N + 1) >= (1ll << 31))
    return SV_ERR_INVALID_ARG;
  if (!cost || !num_draft || !offsets) return SV_ERR_INVALID_ARG;
  if (N > 0 && (!conf || !draft_tokens || !tokens_out)) return SV_ERR_INVALID_ARG;
  AdaptArgs a;
  a.B = B;
  a.N = N;
  a.conf = conf;
  a.cost = cost;
  a.tokens = draft_tokens;
  a.num_draft = num_draft;
  a.offsets = offsets;
  a.tokens_out = tokens_out;
  a.src_index = src_index;
  a.progress = progress;
  (void)hipGetLastError();
  k_adaptive<<<1, kPlanThreads, 0, static_cast<hipStream_t>(stream)>>>(a);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}

extern "C" int32_t spec_verify_gather_rows(int32_t dtype, int32_t V, const void* src,
                                           int64_t src_ld, int32_t src_rows, const int32_t* index,
                                           const int32_t* count, int32_t max_rows, void* dst,
                                           int64_t dst_ld, void* stream) {
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_UNSUPPORTED;
  const int es = dtype == SV_F32 ? 4 : 2;
  if (V < 1 || V > (1 << 30) || max_rows < 0 || src_rows < 0) return SV_ERR_INVALID_ARG;
  if (src_ld < V || dst_ld < V || src_ld > (1ll << 40) || dst_ld > (1ll << 40)) return SV_ERR_INVALID_ARG;
  if (!src || !dst || !index || !count) return SV_ERR_INVALID_ARG;
  if ((uintptr_t)src % es != 0 || (uintptr_t)dst % es != 0) return SV_ERR_INVALID_ARG;
  if (max_rows == 0) return SV_OK;
  GatherArgs g;
  g.V = V;
  g.max_rows = max_rows;
  g.src_rows = src_rows;
  g.es = es;
  g.src_ld = src_ld;
  g.dst_ld = dst_ld;
  g.src = static_cast<const uint8_t*>(src);
  g.dst = static_cast<uint8_t*>(dst);
  g.index = index;
  g.count = count;
  g.vec = ((uintptr_t)src % 16 == 0) && ((uintptr_t)dst % 16 == 0) && ((src_ld * es) % 16 == 0) &&
          ((dst_ld * es) % 16 == 0);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SV_ERR_HIP;
  const long long pieces = ((long long)V * es + 32767) / 32768;
  const long long units = (long long)max_rows * pieces;
  const long long cus = cu_count(dev);
  const int grid = (int)std::max(1ll, std::min(cus * kBlocksPerCU, (units + kWavesPerBlock - 1) / kWavesPerBlock));
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (g_ev_begin && g_ev_end) (void)hipEventRecord((hipEvent_t)g_ev_begin, st);
  k_gather_rows<<<grid, kBlock, 0, st>>>(g);
  if (g_ev_begin && g_ev_end) (void)hipEventRecord((hipEvent_t)g_ev_end, st);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}
