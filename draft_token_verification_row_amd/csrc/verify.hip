// verify.hip - one-round draft-token verification for AMD Instinct MI355X (gfx950):
// the all-rows, single-launch and early-exit pipelines.
//
// Implements the C ABI of include/spec_verify.h.  The operation is the
// verification step of one speculative-decoding round (chzhyang, "Speculative
// Decoding: Medusa, MTP, EAGLE, DFlash, DDTree, and DSpark", section 1; vLLM blog
// "speculative-decoding-amd-gpus", "Core idea of speculative decoding").
//
// All-rows pipeline (spec_verify_greedy / spec_verify_sample; every launch on
// the caller's stream, no host synchronisation):
//   k_stats     persistent grid, one wavefront per 32 KiB slice ("unit") of a
//               row.  Each workgroup first plans the call in LDS (exclusive
//               scan of num_draft, the table of logit rows to read: every
//               target row, the draft rows of stochastic requests); workgroup 0
//               also writes the request records and the list of stochastic
//               requests.  Then it streams the logits once from HBM with
//               16-byte loads and writes per-unit partials: online max and sum
//               of exp((z-max)/T) for softmax rows, (max, lowest id) for greedy
//               rows.  This is the HBM-bound kernel that carries almost all
//               bytes.  (k_plan writes the same plan to the workspace first
//               when a call has more requests or rows than the LDS table holds.)
//   k_resid     persistent grid over the residual units of the stochastic
//               requests.  A wavefront first decides the request its units
//               belong to (decide_request: combines the partials of each row,
//               evaluates p(y_i), q(y_i) in fp64, runs the ratio tests left to
//               right, cuts at the first rejection; the wavefront holding the
//               request's first unit writes its outputs), then, if the request
//               was cut by a rejection, sums [p - q]_+ over its units of the
//               rejected (target, draft) row pair.
//   k_finalize  one workgroup per request: the decision of a greedy request
//               (the argmax tests and the target's token), or the draw of a
//               stochastic one: finds the unit holding the inverse-CDF crossing
//               from the unit sums (bonus: from the k_stats partials, no
//               re-read), rescans that unit only, keeps the fp32 draw when its
//               margin certifies it and otherwise redoes it in fp64.
// Small calls run all of this in one launch instead (k_fused, one workgroup
// per request).
//
// Early-exit pipeline (the *_early_exit entry points): k_plan_ee, then per
// window of positions a k_round launch (row statistics of the window's rows
// of the requests still undecided, residual sweeps of the requests cut in the
// previous window) and a k_decide_round launch (decides the window), one more
// k_round for the last window's residual sweeps, then k_finalize.
//
// Numerics.  Every exponent is exp2((z - m) * c) with one fp32 scale
// c = fl(log2(e)/T): all kernels compute the softmax at the temperature
// log2(e)/c, within a relative 2^-24 of T.  Lane partial sums are fp32 over at
// most a few dozen terms, combined across lanes, units and rows in fp64.  p(y)
// and q(y) are formed in fp64 as exp2((z_y - M) * c) / S (the product is exact
// in fp64).  A stochastic row whose logits are all -inf has no distribution:
// a request that tests such a row reports -1.  Greedy argmax is exact
// (lexicographic max of (value, -id)).
#include "sv_common.hpp"

#include <mutex>

namespace {

// ------------------------------------------------------------------ k_plan

// One workgroup: the plan of a call too large for k_stats to plan in LDS
// (plan_fits_lds): exclusive scan of k_b -> request offsets and
// records, the list of stochastic requests, and the two row lists k_stats
// streams (row_counts, row_in_first, row_in_second), 1024 requests per pass
// (wave shuffles + one LDS step).
__global__ __launch_bounds__(kPlanThreads) void k_plan(Args a) {
  constexpr int kPlanWaves = kPlanThreads / kWave;
  __shared__ long long s_w0[kPlanWaves];
  __shared__ long long s_w1[kPlanWaves];
  __shared__ long long s_tot[2];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  const long long TB = (long long)a.K + a.B;
  long long carry_k = 0, carry_a = 0, carry_b = 0, carry_s = 0;
  for (int base = 0; base < a.B; base += kPlanThreads) {
    const int b = base + tid;
    int k = 0;
    bool g = true;
    if (b < a.B) {
      k = a.num_draft[b];
      if (k < 0 || k > a.K) {
        s_bad = 1;
        k = 0;
      }
      g = a.force_greedy ? true : (a.gmask ? (a.gmask[b] != 0) : false);
    }
    int cA = 0, cB = 0;
    if (b < a.B) row_counts(k, g, cA, cB);
    const Scan2 sc = block_scan2(k, cA, s_w0, s_w1, s_tot);
    __syncthreads();
    const Scan2 sb = block_scan2(cB, (b < a.B && !g) ? 1 : 0, s_w0, s_w1, s_tot);
    const long long off = carry_k + sc.ex0;
    const long long aoff = carry_a + sc.ex1;
    const long long boff = carry_b + sb.ex0;
    const long long soff = carry_s + sb.ex1;
    if (b < a.B) {
      ReqInfo r;
      r.off = (int)off;
      r.k = k;
      r.greedy = g ? 1 : 0;
      r.a = 0;
      r.kind = KIND_NONE;
      r.y = -1;
      r.trow = -1;
      r.drow = -1;
      r.Mp = r.Mq = 0.f;
      r.pad0 = r.pad1 = 0;
      r.Sp = r.Sq = 0.0;
      a.ws.req[b] = r;
      if (!g && soff < a.B) a.ws.stoch_list[soff] = b;
      // (offsets are wrong when num_draft is inconsistent: the call is then
      // reported as an error, and every write stays inside its list)
      if (off + b + k < TB)
        for (int j = 0; j < cA; ++j)
          if (aoff + j < 2ll * a.K + a.B) a.ws.rowdesc[aoff + j] = row_in_first(b, j, (int)off, k, g);
      if (off < a.K)
        for (int j = 0; j < cB; ++j)
          if (boff + j < 2ll * a.B) a.ws.rowdesc_b[boff + j] = row_in_second(b, j, (int)off);
    }
    carry_k += sc.tot0;
    carry_a += sc.tot1;
    carry_b += sb.tot0;
    carry_s += sb.tot1;
    __syncthreads();
  }
  if (tid == 0) {
    const bool bad = s_bad != 0 || carry_k != a.K;
    Header* h = a.ws.hdr;
    h->error = bad ? 1 : 0;
    h->n_rows = bad ? 0 : (int)carry_a;
    h->n_rows_b = bad ? 0 : (int)carry_b;
    h->n_stoch = bad ? 0 : (int)carry_s;
    h->n_units = 0;
  }
}

// ------------------------------------------------------------------ row combines
// One lane combines the nseg unit partials of one row.  Loads are issued in
// groups of 16 so that they are in flight together (one group covers a
// 262144-id bf16 row); unit factors use the same scaled exp2 as the streaming
// kernels and accumulate in fp64.
constexpr int kCombineGroup = 16;

__device__ void row_softmax(const Partial* P, int nseg, float c, float& M, double& S) {
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
      s *= (double)scaled_exp(m - gm, c);
      m = gm;
    }
#pragma unroll
    for (int j = 0; j < kCombineGroup; ++j)
      if (ps[j] > 0.0) s += ps[j] * (double)scaled_exp(pm[j] - m, c);
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

// ------------------------------------------------------------------ decisions
// Decision of every position of request b by one wavefront, from the row
// partials in the workspace and R, the request's plan record (offset, k_b,
// greedy).  Positions are taken 32 at a time: lane l < 32 combines the target
// row of position base+l, lane l+32 the draft row of the same position, so
// every row of a request is combined in parallel.  Returns the decision record
// (cut, final row, and for stochastic requests the statistics of the rows the
// draw needs), the same in every lane.  write: also write the request's
// outputs (accepted length, kept drafts, greedy target token, p(y), q(y), -1
// slots) and its record; several wavefronts may compute the same decision, and
// exactly one of them writes.
template <class D>
__device__ __forceinline__ ReqInfo decide_request(const Args& a, int b, int lane, bool write,
                                                  const ReqInfo& R) {
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
  bool no_mass = false;     // a row at a position <= A has no mass (all -inf)
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
        row_softmax(P, nseg, a.c, M, S);
    } else if (upper && !g && i < k) {
      row_softmax(a.ws.pd + (int64_t)(drow0 + i) * nseg, nseg, a.c, M, S);
    }
    const float Mq = __shfl(M, half + 32);
    const double Sq = __shfl(S, half + 32);
    const bool own_ok = g || row_has_mass(S);
    const bool draft_ok = __shfl(own_ok, half + 32);
    const bool pos_ok = own_ok && (i >= k || draft_ok);    // lanes < 32, positions i <= k
    const bool was_found = found;
    bool rej = false;
    if (!upper && i < k) {
      if (g) {
        rej = (y != amax);
      } else if (!yok) {
        invalid = true;  // every output of the request becomes -1 below
      } else if (!pos_ok) {
        rej = true;      // a row without mass: -1 here (the request is invalid if tested)
        if (write && a.p_out) a.p_out[drow0 + i] = -1.f;
        if (write && a.q_out) a.q_out[drow0 + i] = -1.f;
      } else {
        const double py = exp2(((double)zy - (double)M) * a.c64) / S;
        const double qy = exp2(((double)dy - (double)Mq) * a.c64) / Sq;
        rej = !((double)a.u_accept[drow0 + i] * qy < py);
        if (write && a.p_out) a.p_out[drow0 + i] = (float)py;
        if (write && a.q_out) a.q_out[drow0 + i] = (float)qy;
      }
    }
    const unsigned long long rm = __ballot(rej);
    if (!found && rm != 0ull) {
      A = base + __ffsll((long long)rm) - 1;
      found = true;
    } else if (!found && k < base + 32) {
      found = true;      // A = k, the bonus row lies in this chunk
    }
    if (!was_found) {    // positions base .. min(A, base + 31) are tested
      const unsigned long long bad = __ballot(!upper && i <= k && !pos_ok);
      const unsigned long long tested =
          found ? ((A - base >= 63) ? ~0ull : ((2ull << (A - base)) - 1ull)) : ~0ull;
      if (bad & tested) no_mass = true;
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
  ReqInfo W = R;
  if (__any(invalid) || no_mass) {
    W.kind = KIND_INVALID;
    if (write) {
      for (int i = lane; i <= k; i += kWave) a.out[trow0 + i] = -1;
      for (int i = lane; i < k; i += kWave) {
        if (a.p_out) a.p_out[drow0 + i] = -1.f;
        if (a.q_out) a.q_out[drow0 + i] = -1.f;
      }
      if (lane == 0) {
        a.acc_len[b] = -1;
        if (a.resid_out) a.resid_out[b] = -1.f;
        a.ws.req[b] = W;
      }
    }
    return W;
  }
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
    } else {
      W.kind = KIND_BONUS;
      W.drow = -1;
      W.y = -1;
    }
  }
  if (!write) return W;
  if (g) {
    // no probabilities for greedy rows: every position, also those after the
    // cut that the loop above never reached
    for (int i = lane; i < k; i += kWave) {
      if (a.p_out) a.p_out[drow0 + i] = -1.f;
      if (a.q_out) a.q_out[drow0 + i] = -1.f;
    }
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
    a.ws.req[b] = W;
  }
  return W;
}


// Every output slot of a call whose num_draft is inconsistent becomes -1;
// thread gt of gs threads in all takes its share.
__device__ __forceinline__ void fill_error_outputs(const Args& a, long long gt, long long gs) {
  for (long long i = gt; i < (long long)a.K + a.B; i += gs) a.out[i] = -1;
  for (long long i = gt; i < a.B; i += gs) {
    a.acc_len[i] = -1;
    if (a.resid_out) a.resid_out[i] = -1.f;
  }
  for (long long i = gt; i < a.K; i += gs) {
    if (a.p_out) a.p_out[i] = -1.f;
    if (a.q_out) a.q_out[i] = -1.f;
  }
}

// ------------------------------------------------------------------ draw weights
// Residual weight [p - q]_+ and target weight p of one id, from the exact row
// maxima and the row sums.  The residual sweep accumulates raw() =
// S_p [p - q]_+ = [exp2((z - M_p) c) - rho exp2((d - M_q) c)]_+ with
// rho = fl(S_p / S_q) and applies 1/S_p once per unit in fp64; single ids
// (the rescan of one unit) use raw() times fl(1/S_p).
struct ResidW {
  float Mp, Mq, rho, ip, c;
  double ip64;
  __device__ __forceinline__ float raw(float z, float d) const {
    return fmaxf(fmaf(-scaled_exp(d - Mq, c), rho, scaled_exp(z - Mp, c)), 0.f);
  }
  __device__ __forceinline__ float operator()(float z, float d) const { return raw(z, d) * ip; }
};

struct TargetW {
  float Mp, ip, c;
  __device__ __forceinline__ float operator()(float z) const {
    return scaled_exp(z - Mp, c) * ip;
  }
};

__device__ __forceinline__ ResidW resid_weights(const ReqInfo& R, const Args& a) {
  ResidW w;
  w.Mp = R.Mp;
  w.Mq = R.Mq;
  w.rho = (float)(R.Sp / R.Sq);
  w.ip64 = 1.0 / R.Sp;
  w.ip = (float)w.ip64;
  w.c = a.c;
  return w;
}

__device__ __forceinline__ TargetW target_weights(const ReqInfo& R, const Args& a) {
  TargetW w;
  w.Mp = R.Mp;
  w.ip = (float)(1.0 / R.Sp);
  w.c = a.c;
  return w;
}

// Sum of [p - q]_+ over the ids [s0, s1) of one (target, draft) row pair, the
// rejected id y excluded; one wavefront, result in every lane.  Lane l takes
// the 16-byte chunks l, l + 64, ... in order; the loop is software-pipelined
// over two register sets (the U chunks of both rows for the next step are
// requested before the current ones are consumed, with no copies between the
// sets), so any U gives the same sums bit for bit.
template <class L, int U>
__device__ __forceinline__ double resid_unit(const typename L::Elem* tp, const typename L::Elem* dp,
                                             const ResidW& fw, int y, int s0, int s1, int lane) {
  constexpr int E = L::E;
  using Raw = typename L::Raw;
  const int n = s1 - s0;
  const int nchunk = n / E;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  auto consume = [&](const Raw* rt, const Raw* rd) {
#pragma unroll
    for (int jj = 0; jj < U; ++jj) {
      float vt[E], vd[E];
      L::unpack(rt[jj], vt);
      L::unpack(rd[jj], vd);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += fw.raw(vt[e], vd[e]);
    }
  };
  auto load = [&](Raw* rt, Raw* rd, int c0) {
#pragma unroll
    for (int jj = 0; jj < U; ++jj) {
      rt[jj] = L::stream(tp + s0 + (size_t)(c0 + jj * kWave) * E);
      rd[jj] = L::stream(dp + s0 + (size_t)(c0 + jj * kWave) * E);
    }
  };
  constexpr int per_it = kWave * U;
  const int nit = nchunk / per_it;
  int c = lane;
  if (nit > 0) {
    Raw at[U], ad[U], bt[U], bd[U];
    load(at, ad, c);
    int it = 1;
    for (; it + 1 < nit; it += 2) {
      load(bt, bd, c + per_it);
      consume(at, ad);
      c += per_it;
      load(at, ad, c + per_it);
      consume(bt, bd);
      c += per_it;
    }
    if (it < nit) {
      load(bt, bd, c + per_it);
      consume(at, ad);
      c += per_it;
      consume(bt, bd);
    } else {
      consume(at, ad);
    }
    c += per_it;
  }
  for (; c < nchunk; c += kWave) {
    Raw rt = L::stream(tp + s0 + (size_t)c * E), rd = L::stream(dp + s0 + (size_t)c * E);
    float vt[E], vd[E];
    L::unpack(rt, vt);
    L::unpack(rd, vd);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += fw.raw(vt[e], vd[e]);
  }
  const int tail0 = nchunk * E;
  if (lane < n - tail0) {
    const int v = s0 + tail0 + lane;
    acc[0] += fw.raw(L::one(tp + v), L::one(dp + v));
  }
  // The rejected id y carries no residual weight (rejection means p(y) < q(y),
  // so [p - q]_+ is 0 there), but its fp32 weight can round above 0: the lane
  // that accumulated it takes the same value back out (y is the same in every
  // lane, so the loop above has no per-id test).
  if (y >= s0 && y < s1) {
    const int rel = y - s0;
    const bool chunked = rel < tail0;
    const int owner = chunked ? (rel / E) & (kWave - 1) : rel - tail0;
    const int slot = chunked ? rel % E : 0;
    if (lane == owner) {
      const float ry = fw.raw(L::one(tp + y), L::one(dp + y));
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (e == slot) acc[e] -= ry;
    }
  }
  float sl = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) sl += acc[e];
  return wave_sum((double)sl) * fw.ip64;
}

// ------------------------------------------------------------------ k_resid
// Persistent grid over the residual units of the stochastic requests (nrseg
// units of rseg ids of each request's rejected row pair; the list of
// stochastic requests comes from the plan).  Each wavefront takes a
// contiguous range of units, so its units mostly belong to one request, and
// it decides that request itself (decide_request over the row partials of
// k_stats) before sweeping: the decision needs no launch of its own.  The
// wavefront whose range holds a request's unit 0 also writes the request's
// outputs and record; a request cut at no position (bonus) or invalid has
// nothing to sweep.
template <class L>
__global__ __launch_bounds__(kBlock) void k_resid(Args a) {
  using Elem = typename L::Elem;
  if (a.ws.hdr->error) return;          // k_finalize writes the -1 outputs
  const int lane = threadIdx.x & (kWave - 1);
  const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int W = gridDim.x * kWavesPerBlock;
  const long long n_units = (long long)a.ws.hdr->n_stoch * a.nrseg;
  const int u_begin = (int)(n_units * gw / W);
  const int u_end = (int)(n_units * (gw + 1) / W);
  int cur = -1, b = 0;
  ReqInfo D;
  ResidW fw;
  const Elem* tp = nullptr;
  const Elem* dp = nullptr;
  for (int u = u_begin; u < u_end; ++u) {
    const int j = u / a.nrseg;
    const int seg = u - j * a.nrseg;
    if (j != cur) {
      cur = j;
      b = a.ws.stoch_list[j];
      const ReqInfo R = a.ws.req[b];
      D = decide_request<L>(a, b, lane, (long long)j * a.nrseg >= u_begin, R);
      if (D.kind == KIND_RESID) {
        fw = resid_weights(D, a);
        tp = static_cast<const Elem*>(a.target) + (int64_t)D.trow * a.tld;
        dp = static_cast<const Elem*>(a.draft) + (int64_t)D.drow * a.dld;
      }
    }
    if (D.kind != KIND_RESID) continue;
    const int s0 = seg * a.rseg;
    const int s1 = min(s0 + a.rseg, a.V);
    const double tot = resid_unit<L, kResidUnroll>(tp, dp, fw, D.y, s0, s1, lane);
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
  float Mp, c;
  double invSp;
  bool resid;
  __device__ __forceinline__ double operator()(int s) const {
    if (resid) return rp[s];
    const Partial p = prow[s];
    // the factor is formed whether or not the unit has mass, so that both
    // fields of the partial are requested together (a unit without mass,
    // s = 0, weighs 0; its m of -FLT_MAX gives a factor of 0, never NaN)
    const double f = (double)scaled_exp(p.m - Mp, c);
    return p.s > 0.0 ? p.s * f * invSp : 0.0;
  }
};

// Wave 0 finds the unit holding the crossing of w * Z.  Returns (in lane 0's
// view, broadcast) the unit, the cumulative mass before it and a fallback flag.
// m0_pre: the masses of units 0..63 already loaded by the caller (0 past nunits).
__device__ void find_unit(const UnitMass& um, int nunits, double w, int lane, double& Z,
                          int& unit, double& before, int& fallback,
                          const double* m0_pre = nullptr) {
  // Z is the total of the same chunked scan that locates the crossing, so the
  // two agree bit for bit; with <= 64 units (the usual case) masses load once.
  double m0 = m0_pre ? *m0_pre : ((lane < nunits) ? um(lane) : 0.0);
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

// Weights of the ids [id0, id0 + E) from their logits vt (target) and vd
// (draft; residual weights only), 0 past s1 and at y.
template <class L, class WF>
__device__ __forceinline__ void chunk_weights(const float* vt, const float* vd, int id0, int s1,
                                              int y, const WF& wf, float* w) {
#pragma unroll
  for (int e = 0; e < L::E; ++e) {
    float x;
    if constexpr (std::is_same<WF, ResidW>::value) x = wf(vt[e], vd[e]);
    else x = wf(vt[e]);
    w[e] = (id0 + e < s1 && id0 + e != y) ? x : 0.f;
  }
}

// Weights of the ids [id0, id0 + E) of a unit ending at s1 (0 past s1 and at y),
// loading them element by element where the chunk crosses s1.
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
  chunk_weights<L>(vt, vd, id0, s1, y, wf, w);
}

// The chunks of one thread's span [v0, v0 + PER) that lies wholly before s1,
// requested together (one load latency for the span instead of one per chunk).
template <class L, int PER, bool RESID>
struct SpanRaw {
  typename L::Raw t[PER / L::E];
  typename L::Raw d[RESID ? PER / L::E : 1];
  __device__ __forceinline__ void load(const typename L::Elem* tp, const typename L::Elem* dp,
                                       int v0) {
#pragma unroll
    for (int c = 0; c < PER / L::E; ++c) {
      t[c] = L::load(tp + v0 + c * L::E);
      if constexpr (RESID) d[c] = L::load(dp + v0 + c * L::E);
    }
  }
  template <class WF>
  __device__ __forceinline__ void weights(int c, int id0, int s1, int y, const WF& wf,
                                          float* w) const {
    float vt[L::E], vd[L::E];
    L::unpack(t[c], vt);
    if constexpr (RESID) L::unpack(d[c], vd);
    chunk_weights<L>(vt, vd, id0, s1, y, wf, w);
  }
};

// Rescan one unit of PER * kBlock ids: thread t (< kBlock) sums the weights of
// its PER ids in ascending order, a block-wide exclusive scan of those sums
// locates the crossing thread, which walks its ids again.  KEEP holds the
// weights in registers for that walk; otherwise they are recomputed (same
// values, fewer registers).  In a block larger than kBlock the extra threads
// take part in the barriers only, so the result is the same for any block size.
// The thread that returns the token also stores in *margin the distance of
// thr from the nearer edge of that token's cumulative interval (in the units of
// the weights), or -1 when no id crossed thr and the last id with weight was
// taken instead.
template <class L, int PER, bool KEEP, class WF>
__device__ int rescan_unit(const typename L::Elem* tp, const typename L::Elem* dp, int s0,
                           int s1, int y, const WF& wf, double before, double thr, int fallback,
                           double* s_wave, int* s_owner, double* margin) {
  constexpr int E = L::E;
  static_assert(PER % E == 0, "per-thread ids must be whole chunks");
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid >> 6;
  constexpr bool kResid = std::is_same<WF, ResidW>::value;
  const bool active = tid < kBlock;
  const int v0 = s0 + tid * PER;
  // every thread's span lies wholly before s1 except where the unit ends:
  // there chunks load one by one (and always on unaligned rows, whose
  // one-element chunks would take a register per id)
  const bool whole = L::E > 1 && v0 + PER <= s1;
  float keep[KEEP ? PER : 1];
  SpanRaw<L, PER, kResid> raw;
  double ts = 0.0;
  if (active) {
    if (whole) raw.load(tp, dp, v0);
#pragma unroll
    for (int c = 0; c < PER / E; ++c) {
      float w[E];
      if (whole)
        raw.weights(c, v0 + c * E, s1, y, wf, w);
      else
        unit_weights<L>(tp, dp, v0 + c * E, s1, y, wf, w);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        ts += (double)w[e];
        if constexpr (KEEP) keep[c * E + e] = w[e];
      }
    }
  }
  // weights of chunk c for the walks below (without KEEP, the walking thread
  // requests its span again first: reload())
  auto reload = [&]() {
    if constexpr (!KEEP) {
      if (whole) raw.load(tp, dp, v0);
    }
  };
  auto chunk = [&](int c, float* w) {
    if constexpr (KEEP) {
#pragma unroll
      for (int e = 0; e < E; ++e) w[e] = keep[c * E + e];
    } else {
      if (whole)
        raw.weights(c, v0 + c * E, s1, y, wf, w);
      else
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
      reload();
      int tok = -1;
#pragma unroll
      for (int c = 0; c < PER / E; ++c) {
        float w[E];
        chunk(c, w);
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (w[e] > 0.f) tok = v0 + c * E + e;
      }
      *margin = -1.0;
      return tok;
    }
    return -2;
  }
  if (tid != owner) return -2;
  reload();
  double cum = excl;
  double lo = 0.0, hi = 0.0;
  int tok = -1, last = -1;
#pragma unroll
  for (int c = 0; c < PER / E; ++c) {
    float w[E];
    chunk(c, w);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const double prev = cum;
      cum += (double)w[e];
      if (w[e] > 0.f) last = v0 + c * E + e;
      if (tok < 0 && cum > thr) {
        tok = v0 + c * E + e;
        lo = prev;
        hi = cum;
      }
    }
  }
  *margin = tok >= 0 ? fmin(thr - lo, hi - thr) : -1.0;
  return tok >= 0 ? tok : last;
}

// ------------------------------------------------------------------ certified draw
// The draw above evaluates the weights in fp32 (exp2 with the fp32 scale c, so
// at the temperature log2(e)/c; reciprocals of the row sums rounded to fp32;
// lane sums of a few dozen fp32 terms) and locates the crossing of w * Z in
// fp64 over them.  Its cumulative masses differ from the exact ones at
// temperature T by about 1e-8 of the probability mass on typical rows; the
// errors of single exp2 evaluations, of the row sums and the 2^-24 relative
// temperature of the fp32 scale keep it below 1e-7 unless a row has extreme
// spread, and below about 1.1e-5 for any row (temperature <= 2 ln(V) 2^-24
// per row, rounding and exp2 <= 2^-20, row sums <= 40 2^-24 relative).
// Contract: the draw equals the exact draw unless the exact crossing lies
// within 1e-6 of the total of the weights from an edge of the chosen id's
// interval (then either neighbour may come back).
//  - a draw from p (bonus) or from a residual whose fp32 total is at least
//    kSmallResidual: an error of 1e-7 of the mass is below 1e-6 of the total,
//    so the fp32 draw keeps the contract;
//  - a residual total below that: the fp32 draw is kept when its crossing
//    lies farther than kCertMargin (above the any-row bound) from both edges;
//  - otherwise, and whenever no id crossed w * Z or the fp32 residual total
//    was 0, the whole workgroup redoes the draw from the logits in fp64:
//    p_v = exp((z_v - M)/T)/S with S summed in fp64, the residual
//    [p_v - q_v]_+ formed from those fp64 values (no cancellation to speak of
//    at any total), its total, and the first id whose running sum exceeds
//    w times that total.  That takes several fp64 passes over the row pair on
//    one CU; it happens only for rows where p and q nearly agree.
constexpr double kSmallResidual = 0.125;
constexpr double kCertMargin = 0x1p-15;
struct FinalizeShared {
  double wave[kWavesPerBlock];
  double before, thr, Z;
  int unit, mode, fallback, owner;
  int tok, cert;                  // the fp32 draw and whether its margin certifies it
  double red[kWavesPerBlock];     // fp64 draw: wave totals of a block scan or sum
  int ptok, found, plast;
};

// Sum of x over the first kBlock threads of the workgroup, in the same order
// in every thread and for any workgroup size (threads past kBlock take part
// in the barriers only).
__device__ double block_sum(double x, double* red) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  x = wave_sum(x);
  __syncthreads();                      // red may still be read by an earlier call
  if (lane == 0 && wv < kWavesPerBlock) red[wv] = x;
  __syncthreads();
  double t = 0.0;
  for (int q = 0; q < kWavesPerBlock; ++q) t += red[q];
  return t;
}

// fp64 weight of one id: p_v, or [p_v - q_v]_+ when dp rows are given.
struct PreciseW {
  double Mp, Mq, Sp, Sq, T;
  bool resid;
  __device__ __forceinline__ double operator()(float z, float d) const {
    const double p = exp(((double)z - Mp) / T) / Sp;
    if (!resid) return p;
    const double q = exp(((double)d - Mq) / T) / Sq;
    return fmax(p - q, 0.0);
  }
};

// Visit the ids [v0, v0 + n) of a target row (and of a draft row when dp is
// not null) in ascending order: f(id, z, d).  Whole chunks use the vector
// loads of L (v0 a multiple of L::E), the rest single elements.
template <class L, class F>
__device__ __forceinline__ void visit_ids(const typename L::Elem* tp, const typename L::Elem* dp,
                                          int v0, int n, F& f) {
  constexpr int E = L::E;
  int v = v0;
  for (; v + E <= v0 + n; v += E) {
    float vt[E], vd[E];
    L::unpack(L::load(tp + v), vt);
    if (dp) L::unpack(L::load(dp + v), vd);
#pragma unroll
    for (int e = 0; e < E; ++e) f(v + e, vt[e], dp ? vd[e] : 0.f);
  }
  for (; v < v0 + n; ++v) f(v, L::one(tp + v), dp ? L::one(dp + v) : 0.f);
}

// The draw in fp64 by the workgroup (every thread calls it; the result is
// valid in every thread).  The ids are split over the first kBlock threads
// whatever the workgroup size, so every launch plan sums in the same order.
// resid: weights [p - q]_+ (falling back to p if their total is 0), else p.
// Returns the token; *Z = total of the residual weights (0 after the
// fallback) or of p.
template <class L>
__device__ int precise_draw(const typename L::Elem* tp, const typename L::Elem* dp, int V,
                            double Mp, double Mq, double T, double w, bool resid, double* Z,
                            FinalizeShared& sh) {
  constexpr int E = L::E;
  constexpr int SLOT = E * 4;           // consecutive ids per thread and tile
  const int tid = threadIdx.x;
  const int nthr = kBlock;              // threads with work; the others idle
  const bool active = tid < nthr;
  const int lane = tid & (kWave - 1);
  const int wv = tid >> 6;
  const int nslot = (V + SLOT - 1) / SLOT;
  // row sums
  PreciseW pw;
  pw.Mp = Mp;
  pw.Mq = Mq;
  pw.T = T;
  double sp = 0.0, sq = 0.0;
  auto sums = [&](int, float z, float d) {
    sp += exp(((double)z - Mp) / T);
    if (resid) sq += exp(((double)d - Mq) / T);
  };
  for (int sl = tid; active && sl < nslot; sl += nthr)
    visit_ids<L>(tp, resid ? dp : nullptr, sl * SLOT, min(SLOT, V - sl * SLOT), sums);
  pw.Sp = block_sum(sp, sh.red);
  pw.Sq = resid ? block_sum(sq, sh.red) : 1.0;
  // totals of the residual and of p
  pw.resid = resid;
  double tr = 0.0, tq = 0.0;
  PreciseW pp = pw;
  pp.resid = false;
  auto totals = [&](int, float z, float d) {
    tq += pp(z, d);
    if (resid) tr += pw(z, d);
  };
  for (int sl = tid; active && sl < nslot; sl += nthr)
    visit_ids<L>(tp, resid ? dp : nullptr, sl * SLOT, min(SLOT, V - sl * SLOT), totals);
  const double Ptot = block_sum(tq, sh.red);
  double total = Ptot;
  if (resid) {
    const double Ztot = block_sum(tr, sh.red);
    if (Ztot > 0.0) total = Ztot;
    else pw.resid = false;              // p == q: draw from p
    *Z = Ztot > 0.0 ? Ztot : 0.0;
  } else {
    *Z = Ptot;
  }
  const double thr = w * total;
  // first id whose running sum exceeds thr, tile by tile (nthr slots a tile)
  if (tid == 0) {
    sh.found = 0;
    sh.plast = -1;
  }
  double carry = 0.0;
  int mylast = -1;
  for (int base = 0; base < nslot; base += nthr) {
    const int sl = base + tid;
    double ts = 0.0;
    int tl = -1;
    auto acc = [&](int v, float z, float d) {
      const double x = pw(z, d);
      ts += x;
      if (x > 0.0) tl = v;
    };
    if (active && sl < nslot)
      visit_ids<L>(tp, pw.resid ? dp : nullptr, sl * SLOT, min(SLOT, V - sl * SLOT), acc);
    if (tl >= 0) mylast = tl;
    const double iw = wave_incl_scan(ts, lane);
    __syncthreads();
    if (lane == kWave - 1 && wv < kWavesPerBlock) sh.red[wv] = iw;
    if (tid == 0) sh.owner = INT_MAX;
    __syncthreads();
    double pre = 0.0, tile = 0.0;
    for (int q = 0; q < kWavesPerBlock; ++q) {
      if (q < wv) pre += sh.red[q];
      tile += sh.red[q];
    }
    const double prev = __shfl_up(iw, 1);
    const double excl = carry + pre + (lane == 0 ? 0.0 : prev);
    const double incl = carry + pre + iw;
    if (active && sl < nslot && incl > thr && ts > 0.0) atomicMin(&sh.owner, tid);
    __syncthreads();
    if (tid == sh.owner) {
      double cum = excl;
      int tok = -1;
      auto walk = [&](int v, float z, float d) {
        const double x = pw(z, d);
        cum += x;
        if (tok < 0 && cum > thr) tok = v;
      };
      visit_ids<L>(tp, pw.resid ? dp : nullptr, sl * SLOT, min(SLOT, V - sl * SLOT), walk);
      sh.ptok = tok >= 0 ? tok : tl;    // rounding: the last id with weight of this slot
      sh.found = 1;
    }
    __syncthreads();
    if (sh.found) break;
    carry += tile;
  }
  if (!sh.found) {                      // w * total at or past the end: last id with weight
    if (mylast >= 0) atomicMax(&sh.plast, mylast);
    __syncthreads();
    if (tid == 0) sh.ptok = sh.plast;
  }
  __syncthreads();
  return sh.ptok;
}


// Correction or bonus draw of request b by one block of >= kBlock threads
// (KEEP: see rescan_unit).
// The request record R, the uniform w and (wave 0, lane l) the residual mass
// of unit l (rp_pre; 0 past nrseg) are loaded by the caller, so that they can
// be requested together.
template <class L, bool KEEP>
__device__ __forceinline__ void finalize_request(const Args& a, int b, const ReqInfo& R, double w,
                                                 double rp_pre, FinalizeShared& sh) {
  using Elem = typename L::Elem;
  constexpr int PER_S = kSegBytes / (int)sizeof(Elem) / kBlock;    // k_stats unit
  constexpr int PER_R = kRSegBytes / (int)sizeof(Elem) / kBlock;   // k_resid unit
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  if (R.kind != KIND_RESID && R.kind != KIND_BONUS) return;
  if (tid < kWave) {
    UnitMass um;
    um.rp = a.ws.rp + (int64_t)b * a.nrseg;
    um.prow = a.ws.pt + (int64_t)R.trow * a.nseg;
    um.Mp = R.Mp;
    um.c = a.c;
    um.invSp = 1.0 / R.Sp;
    um.resid = (R.kind == KIND_RESID);
    int mode = um.resid ? DRAW_RESID : DRAW_FROM_P;
    double Z = 0.0, before = 0.0;
    int unit = 0, fb = 0;
    find_unit(um, um.resid ? a.nrseg : a.nseg, w, lane, Z, unit, before, fb,
              (um.resid && a.nrseg <= kWave) ? &rp_pre : nullptr);
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
      sh.tok = -1;
      sh.cert = 0;
    }
  }
  __syncthreads();
  const int mode = sh.mode;
  const Elem* tp = static_cast<const Elem*>(a.target) + (int64_t)R.trow * a.tld;
  const Elem* dp = (R.kind == KIND_RESID)
                       ? static_cast<const Elem*>(a.draft) + (int64_t)R.drow * a.dld : nullptr;
  int tok;
  double fm = -1.0;
  if (mode == DRAW_RESID) {
    const int s0 = sh.unit * a.rseg;
    const int s1 = min(s0 + a.rseg, a.V);
    tok = rescan_unit<L, PER_R, KEEP>(tp, dp, s0, s1, R.y, resid_weights(R, a), sh.before,
                                      sh.thr, sh.fallback, sh.wave, &sh.owner, &fm);
  } else {
    const int s0 = sh.unit * a.seg;
    const int s1 = min(s0 + a.seg, a.V);
    tok = rescan_unit<L, PER_S, KEEP>(tp, (const Elem*)nullptr, s0, s1, -1,
                                      target_weights(R, a), sh.before, sh.thr, sh.fallback,
                                      sh.wave, &sh.owner, &fm);
  }
  if (tok != -2) {
    sh.tok = tok;
    // (a residual draw that fell back to p because its fp32 total was 0 is
    // never kept: the exact total may be positive)
    const bool crossed = fm >= 0.0;
    const bool resid = R.kind == KIND_RESID;
    sh.cert = (crossed && !(resid && mode != DRAW_RESID) &&
               (!resid || sh.Z >= kSmallResidual || fm > kCertMargin)) ? 1 : 0;
  }
  __syncthreads();
  if (sh.cert) {
    if (tid == 0) {
      a.out[R.trow] = sh.tok;
      if (a.resid_out)
        a.resid_out[b] = (R.kind == KIND_RESID) ? (float)(mode == DRAW_RESID ? sh.Z : 0.0) : -1.f;
    }
    return;
  }
  double Z = 0.0;
  const int ptok = precise_draw<L>(tp, dp, a.V, (double)R.Mp, (double)R.Mq, a.T64, w,
                                   R.kind == KIND_RESID, &Z, sh);
  if (tid == 0) {
    a.out[R.trow] = ptok;
    if (a.resid_out) a.resid_out[b] = (R.kind == KIND_RESID) ? (float)Z : -1.f;
  }
}

// Loads of a draw that depend only on the request index, issued together
// (the residual masses are read whether or not the request has a residual;
// they lie in the workspace either way and are used only for a residual draw).
struct DrawInputs {
  ReqInfo R;
  double w, rp;
};

__device__ __forceinline__ DrawInputs draw_inputs(const Args& a, int b) {
  DrawInputs d;
  const int lane = threadIdx.x & (kWave - 1);
  d.rp = (threadIdx.x < kWave && lane < a.nrseg) ? a.ws.rp[(int64_t)b * a.nrseg + lane] : 0.0;
  d.R = a.ws.req[b];
  d.w = a.u_final ? (double)a.u_final[b] : 0.0;
  return d;
}

// One workgroup per request: the decision of a greedy request (wavefront
// 0), or the correction / bonus draw of a stochastic one; when num_draft is
// inconsistent, every output slot becomes -1 instead.
template <class L>
__global__ __launch_bounds__(kBlock) void k_finalize(Args a) {
  __shared__ FinalizeShared sh;
  const DrawInputs d = draw_inputs(a, blockIdx.x);
  if (a.ws.hdr->error) {
    fill_error_outputs(a, (long long)blockIdx.x * kBlock + threadIdx.x,
                       (long long)gridDim.x * kBlock);
    return;
  }
  if (d.R.greedy) {
    if (threadIdx.x < kWave) decide_request<L>(a, blockIdx.x, threadIdx.x, true, d.R);
    return;
  }
  finalize_request<L, true>(a, blockIdx.x, d.R, d.w, d.rp, sh);
}

// ------------------------------------------------------------------ single-launch path
// Small batches: one workgroup per request runs the whole step (offsets, row
// statistics, decisions, residual sweep, draw) with only block barriers
// between the phases, so a call is one launch instead of three.  Every phase
// calls the same unit, combine, decide and draw code as the multi-kernel
// path, so the results are the same bit for bit, for any workgroup size.
// Workgroups of 1024 threads for fp32 logits; 512 for bf16, whose decision
// and draw code needs more than the 128 registers a 1024-thread workgroup
// leaves each lane (it spilled there, and the 512-thread workgroup measured
// faster on the greedy V = 32000 batch).
template <class L>
constexpr int fused_threads() { return sizeof(typename L::Elem) == 2 ? 512 : 1024; }
constexpr int kFusedMaxWaves = 1024 / kWave;
constexpr int kFusedUnroll = 4;
constexpr int kFusedResidUnroll = 2;

template <class L>
__global__ __launch_bounds__(fused_threads<L>()) void k_fused(Args a) {
  constexpr int kFusedThreads = fused_threads<L>();
  constexpr int kFusedWaves = kFusedThreads / kWave;
  __shared__ FinalizeShared sh;
  __shared__ long long s_pre[kFusedMaxWaves], s_tot[kFusedMaxWaves];
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
  if (wv == 0) decide_request<L>(a, b, lane, true, a.ws.req[b]);
  __syncthreads();
  const ReqInfo R = a.ws.req[b];
  if (R.kind == KIND_RESID) {
    const Elem* tp = tgt + (int64_t)R.trow * a.tld;
    const Elem* dp = drf + (int64_t)R.drow * a.dld;
    const ResidW fw = resid_weights(R, a);
    for (int seg = wv; seg < a.nrseg; seg += kFusedWaves) {
      const int s0 = seg * a.rseg;
      const int s1 = min(s0 + a.rseg, a.V);
      const double t = resid_unit<L, kFusedResidUnroll>(tp, dp, fw, R.y, s0, s1, lane);
      if (lane == 0) a.ws.rp[(int64_t)b * a.nrseg + seg] = t;
    }
    __syncthreads();
  }
  const DrawInputs d = draw_inputs(a, b);
  finalize_request<L, false>(a, b, d.R, d.w, d.rp, sh);
}

// ------------------------------------------------------------------ early exit
// Left-to-right verification that reads the rows only up to a window past each
// request's cut.  Round r covers the positions [P_r, P_(r+1)) with P = 0, 1,
// 2, 4, 8, ... (the last window ends at max_k + 1), so a call is about
// log2(max_k) + 2 rounds instead of one per position; a request cut inside a
// window has had the rest of that window read for nothing (at most as many
// rows as it had kept before the window).  Round r is two launches: k_round
// streams the window's rows of every request still undecided (and the
// residual row pairs of the requests cut in round r - 1), then k_decide_round
// decides those positions in order, up to the first rejection, and lists the
// kept requests with the rows of their next window, and the new residual
// sweeps.  One more k_round sweeps the residuals of the last window's cuts.
// Lists rotate over three buffers; k_round of round r clears the counts of
// the list that k_decide_round of round r fills.  No kernel waits on another
// wavefront: every hand-over is a kernel boundary.

// One workgroup: offsets as in k_plan, every output set to -1 (slots no round
// reaches keep it), round 0 lists every request with its position-0 rows.
__global__ __launch_bounds__(kPlanThreads) void k_plan_ee(Args a) {
  constexpr int kPlanWaves = kPlanThreads / kWave;
  __shared__ long long s_wk[kPlanWaves];
  __shared__ long long s_wr[kPlanWaves];
  __shared__ long long s_tot[2];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
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
    const Scan2 sc = block_scan2(k, nr, s_wk, s_wr, s_tot);
    const long long off = carry_k + sc.ex0;
    const long long roff = carry_r + sc.ex1;
    const long long tot_k = sc.tot0, tot_r = sc.tot1;
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
      AliveEntry e;
      e.b = b;
      e.off = (int)off;
      e.k = (int)k;
      e.greedy = g;
      a.ws.alive_e[b] = e;
      const long long trow = off + b;
      if (roff < 2ll * a.K + a.B && trow < (long long)a.K + a.B)
        a.ws.rows_r[roff] = (uint32_t)trow | (g ? kGreedyBit : 0u);
      if (pair && roff + 1 < 2ll * a.K + a.B && off < a.K)
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
    h->n_stoch = 0;
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

// Decision of the positions [lo, hi) of request b (up to its cut) by one
// wavefront, 32 positions at a time: lane l < 32 combines the target row of
// position base + l and lane l + 32 its draft row, with the per-row combines
// of decide_request, so both paths see the same statistics bit for bit.  A request
// that keeps every position of the window lists the rows of [hi, nhi) for the
// next round; a cut lists the request's residual sweep.
template <class L>
__device__ __forceinline__ void decide_window(const Args& a, const AliveEntry& e, int lo, int hi,
                                              int nhi, int nxt, int lane) {
  Header* hdr = a.ws.hdr;
  const int b = e.b;
  const int k = e.k;
  const bool g = e.greedy != 0;
  const int trow0 = e.off + b;
  const int drow0 = e.off;
  const int nseg = a.nseg;
  const int half = lane & 31;
  const bool upper = lane >= 32;
  if (lo == 0 && !g) {
    // a stochastic request with a draft token outside [0, V) reports -1
    // everywhere, as on the all-rows path: all its tokens are tested up front
    bool bad = false;
    for (int i = lane; i < k; i += kWave) {
      const int y = a.tokens[drow0 + i];
      bad |= (y < 0 || y >= a.V);
    }
    if (__any(bad)) return;             // outputs keep the -1 written by the plan
  }
  const int end = min(hi, k + 1);       // positions lo .. end - 1 (position k: the final token)
  const int dend = min(hi, k);          // positions with a draft token
  int A = -1;                           // cut position, -1 while every position is kept
  bool bonus = false;                   // position k reached: every draft kept
  bool no_mass = false;                 // a tested row has no mass: the request is invalid
  float MpA = 0.f, MqA = 0.f;
  double SpA = 0.0, SqA = 0.0;
  int amaxA = INT_MAX;
  for (int base = lo; base < end && A < 0 && !bonus; base += 32) {
    const int i = base + half;
    // loads that depend only on the request are issued before the row combines
    int y = 0;
    float zy = 0.f, dy = 0.f, u = 0.f;
    if (!upper && i < dend) {
      y = a.tokens[drow0 + i];
      if (!g) {
        u = a.u_accept[drow0 + i];
        if (y >= 0 && y < a.V) {        // checked for every token in the first window
          zy = logit_at<L>(a.target, trow0 + i, a.tld, y);
          dy = logit_at<L>(a.draft, drow0 + i, a.dld, y);
        }
      }
    }
    float M = 0.f;
    double S = 0.0;
    int amax = INT_MAX;
    if (!upper && i < end) {
      const Partial* P = a.ws.pt + (int64_t)(trow0 + i) * nseg;
      if (g)
        row_argmax(P, nseg, amax);
      else
        row_softmax(P, nseg, a.c, M, S);
    } else if (upper && !g && i < dend) {
      row_softmax(a.ws.pd + (int64_t)(drow0 + i) * nseg, nseg, a.c, M, S);
    }
    const float Mq = __shfl(M, half + 32);
    const double Sq = __shfl(S, half + 32);
    const bool own_ok = g || row_has_mass(S);
    const bool draft_ok = __shfl(own_ok, half + 32);
    const bool pos_ok = own_ok && (i >= k || draft_ok);    // lanes < 32, positions i < end
    bool rej = false;
    double py = 0.0, qy = 0.0;
    if (!upper && i < dend) {
      if (g) {
        rej = (y != amax);
      } else if (!pos_ok) {
        rej = true;                     // tested: the request is reported invalid
      } else {
        py = exp2(((double)zy - (double)M) * a.c64) / S;
        qy = exp2(((double)dy - (double)Mq) * a.c64) / Sq;
        rej = !((double)u * qy < py);
      }
    }
    const unsigned long long rm = __ballot(rej);
    int last;                           // last position of this chunk that is tested
    if (rm != 0ull) {
      A = base + __ffsll((long long)rm) - 1;
      last = A;
    } else {
      last = min(end, base + 32) - 1;
      if (last == k) bonus = true;
    }
    if (__ballot(!upper && i <= last && !pos_ok) != 0ull) {
      no_mass = true;
      break;
    }
    if (!upper && i <= last && i < k) {
      if (!g) {
        if (a.p_out) a.p_out[drow0 + i] = (float)py;
        if (a.q_out) a.q_out[drow0 + i] = (float)qy;
      }
      if (i != A) a.out[trow0 + i] = y;  // kept draft
    }
    if (A >= 0 || bonus) {
      const int src = last - base;
      MpA = __shfl(M, src);
      SpA = __shfl(S, src);
      MqA = __shfl(M, src + 32);
      SqA = __shfl(S, src + 32);
      amaxA = __shfl(amax, src);
    }
  }
  if (no_mass) {
    // slots, p and q written by earlier windows are reset as well
    for (int i = lane; i <= k; i += kWave) a.out[trow0 + i] = -1;
    for (int i = lane; i < k; i += kWave) {
      if (a.p_out) a.p_out[drow0 + i] = -1.f;
      if (a.q_out) a.q_out[drow0 + i] = -1.f;
    }
    if (lane == 0) a.acc_len[b] = -1;
    return;
  }
  if (A < 0 && !bonus) {                // every position of the window kept: list [hi, nhi)
    const int nt = min(nhi, k + 1) - hi;
    const int nd = g ? 0 : max(0, min(nhi, k) - hi);
    int ir = 0;
    if (lane == 0) {
      const int ia = atomicAdd(&hdr->n_alive3[nxt], 1);
      a.ws.alive_e[(int64_t)nxt * a.B + ia] = e;
      ir = atomicAdd(&hdr->n_rows3[nxt], nt + nd);
    }
    ir = __shfl(ir, 0);
    uint32_t* rows = a.ws.rows_r + (int64_t)nxt * (2ll * a.K + a.B);
    for (int t = lane; t < nt + nd; t += kWave)
      rows[ir + t] = (t < nt) ? ((uint32_t)(trow0 + hi + t) | (g ? kGreedyBit : 0u))
                              : ((uint32_t)(drow0 + hi + (t - nt)) | kDraftBit);
    return;
  }
  if (lane != 0) return;
  ReqInfo Wr;                           // the record k_round and k_finalize read
  Wr.off = e.off;
  Wr.k = k;
  Wr.greedy = e.greedy;
  Wr.pad0 = Wr.pad1 = 0;
  Wr.Mq = 0.f;
  Wr.Sq = 0.0;
  Wr.y = -1;
  Wr.drow = -1;
  Wr.kind = KIND_NONE;
  if (bonus) {                          // every draft kept: the final token
    a.acc_len[b] = k;
    if (g) {
      a.out[trow0 + k] = (amaxA == INT_MAX) ? -1 : amaxA;
    } else {                            // drawn by k_finalize after the last round
      Wr.a = k;
      Wr.trow = trow0 + k;
      Wr.kind = KIND_BONUS;
      Wr.Mp = MpA;
      Wr.Sp = SpA;
      a.ws.req[b] = Wr;
    }
    return;
  }
  a.acc_len[b] = A;                     // cut at A
  if (g) {
    a.out[trow0 + A] = (amaxA == INT_MAX) ? -1 : amaxA;
  } else {                              // pair swept in the next round, drawn by k_finalize
    Wr.a = A;
    Wr.trow = trow0 + A;
    Wr.drow = drow0 + A;
    Wr.y = a.tokens[drow0 + A];
    Wr.kind = KIND_RESID;
    Wr.Mp = MpA;
    Wr.Sp = SpA;
    Wr.Mq = MqA;
    Wr.Sq = SqA;
    a.ws.req[b] = Wr;
    const int ir = atomicAdd(&hdr->n_res3[nxt], 1);
    a.ws.res_r[(int64_t)nxt * a.B + ir] = b;
  }
}

// Round r (a.ee_round), streaming half: persistent grid over the round's
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
    // the lists k_decide_round of this round fills; round r - 2 read them
    hdr->n_rows3[nxt] = 0;
    hdr->n_res3[nxt] = 0;
    hdr->n_alive3[nxt] = 0;
  }
  const int n_s = hdr->n_rows3[cur] * a.nseg;
  const int n_units = n_s + hdr->n_res3[cur] * a.nrseg;
  const uint32_t* rows = a.ws.rows_r + (int64_t)cur * (2ll * a.K + a.B);
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
    } else {                            // residual unit of a request cut in round r - 1
      const int v = u - n_s;
      const int ri = v / a.nrseg;
      const int seg = v - ri * a.nrseg;
      const int b = res[ri];
      const ReqInfo R = a.ws.req[b];
      const Elem* tp = tgt + (int64_t)R.trow * a.tld;
      const Elem* dp = drf + (int64_t)R.drow * a.dld;
      const int s0 = seg * a.rseg;
      const int s1 = min(s0 + a.rseg, a.V);
      const double tot = resid_unit<L, kRoundResidUnroll>(tp, dp, resid_weights(R, a), R.y, s0, s1, lane);
      if (lane == 0) a.ws.rp[(int64_t)b * a.nrseg + seg] = tot;
    }
  }
}

// Round r, deciding half: one wavefront per request whose window rows the
// round streamed.
template <class L>
__global__ __launch_bounds__(kBlock) void k_decide_round(Args a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int W = gridDim.x * kWavesPerBlock;
  const int j = a.ee_round;
  const int cur = j % 3, nxt = (j + 1) % 3;
  const AliveEntry* list = a.ws.alive_e + (int64_t)cur * a.B;
  // the first entry is loaded together with the count (every index < B is in
  // the buffer; entries at or past the count are not used)
  AliveEntry e;
  if (gw < a.B) e = list[gw];
  const int nal = a.ws.hdr->n_alive3[cur];
  for (int w = gw; w < nal; w += W) {
    if (w != gw) e = list[w];
    decide_window<L>(a, e, a.ee_lo, a.ee_hi, a.ee_nhi, nxt, lane);
  }
}

// ------------------------------------------------------------------ host side

struct Sizes {
  size_t off_hdr, off_req, off_rowdesc, off_rowdesc_b, off_resid, off_pt, off_pd, off_rp,
      off_rows_r, off_res_r, off_alive, total;
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
  z->off_rowdesc_b = o; o = align_up(o + 4 * (size_t)(2 * B), 256);
  z->off_resid = o; o = align_up(o + 4 * (size_t)B, 256);
  z->off_pt = o; o = align_up(o + sizeof(Partial) * (size_t)((K + B) * nseg), 256);
  z->off_pd = o; o = align_up(o + sizeof(Partial) * (size_t)(K * nseg), 256);
  z->off_rp = o; o = align_up(o + sizeof(double) * (size_t)(B * nrseg), 256);
  z->off_rows_r = o; o = align_up(o + 4 * (size_t)(3 * (2 * K + B)), 256);
  z->off_res_r = o; o = align_up(o + 4 * (size_t)(3 * B), 256);
  z->off_alive = o; o = align_up(o + sizeof(AliveEntry) * (size_t)(3 * B), 256);
  z->total = o + 256;   // slack for aligning the caller's pointer
  return true;
}


// Logit bytes up to which a batch runs as one launch (one workgroup per
// request): below this the multi-kernel path is bound by launch latency.
constexpr long long kFusedMaxBytes = 48ll << 20;
constexpr int kFusedMaxRequests = 2048;



// Resident workgroups per CU for a kernel, from the occupancy calculator
// (cached per device); the persistent grids are sized to exactly fill the chip.

template <class L>
void launch_fused(const Args& a, hipStream_t st) {
  if (g_ev_begin && g_ev_end) (void)hipEventRecord((hipEvent_t)g_ev_begin, st);
  k_fused<L><<<a.B, fused_threads<L>(), 0, st>>>(a);
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
  // small enough calls are planned by k_stats itself (the row table in LDS)
  Args sa = a;
  sa.plan_in_kernel = plan_fits_lds(a.B, a.K) ? 1 : 0;
  const size_t lds = sa.plan_in_kernel ? plan_lds_bytes(a.B, a.K) : 0;
  if (!sa.plan_in_kernel) k_plan<<<1, kPlanThreads, 0, st>>>(a);
  if (g_ev_begin && g_ev_end) (void)hipEventRecord((hipEvent_t)g_ev_begin, st);
  k_stats<L><<<grid_stats, kBlock, lds, st>>>(sa);
  if (g_ev_begin && g_ev_end) (void)hipEventRecord((hipEvent_t)g_ev_end, st);
  if (sample) {
    const long long cap_r = cus * resident_blocks(occ_resid, k_resid<L>, dev);
    const int grid_resid = (int)std::max(1ll, std::min(cap_r, (units_resid + kWavesPerBlock - 1) / kWavesPerBlock));
    k_resid<L><<<grid_resid, kBlock, 0, st>>>(a);
  }
  k_finalize<L><<<a.B, kBlock, 0, st>>>(a);
}

template <class L>
void launch_early_exit(const Args& a, hipStream_t st, int dev, bool sample) {
  static std::atomic<int> occ_round[64];
  const long long cus = cu_count(dev);
  const long long units_max = (2ll * a.K + a.B) * a.nseg + (long long)a.B * a.nrseg;
  const long long cap = cus * resident_blocks(occ_round, k_round<L>, dev);
  const int grid = (int)std::max(1ll, std::min(cap, (units_max + kWavesPerBlock - 1) / kWavesPerBlock));
  const int grid_dec = (int)std::max(1ll, std::min(cus * kBlocksPerCU, ((long long)a.B + kWavesPerBlock - 1) / kWavesPerBlock));
  k_plan_ee<<<1, kPlanThreads, 0, st>>>(a);
  if (g_ev_begin && g_ev_end) (void)hipEventRecord((hipEvent_t)g_ev_begin, st);
  // windows [P_r, P_(r+1)) with P = 0, 1, 2, 4, 8, ..., the last one ending at
  // max_k + 1; k_plan_ee lists the rows of the first window (position 0)
  const int end = a.max_k + 1;
  auto start = [](int r) { return r == 0 ? 0 : (1 << (r - 1)); };
  int r = 0;
  int lo = 0;
  while (lo < end) {
    const int hi = std::min(start(r + 1), end);
    Args ra = a;
    ra.ee_round = r;
    ra.ee_lo = lo;
    ra.ee_hi = hi;
    ra.ee_nhi = std::min(start(r + 2), end);
    k_round<L><<<grid, kBlock, 0, st>>>(ra);
    k_decide_round<L><<<grid_dec, kBlock, 0, st>>>(ra);
    if (hi >= end && lo < end - 1) {
      // residual sweeps of the cuts in the last window (no rows are listed)
      ra.ee_round = r + 1;
      k_round<L><<<grid, kBlock, 0, st>>>(ra);
    }
    lo = hi;
    ++r;
  }
  if (g_ev_begin && g_ev_end) (void)hipEventRecord((hipEvent_t)g_ev_end, st);
  if (sample) k_finalize<L><<<a.B, kBlock, 0, st>>>(a);
}

// Host-side checks of a verification call (everything but the workspace);
// they touch no GPU state.  *z receives the workspace layout of the call.
int32_t host_checks(const sv_batch_t* bt, bool sample, float temperature, const float* u_accept,
                    const float* u_final, const int32_t* acc_len, const int32_t* out,
                    bool early_exit, int max_k, Sizes* zp) {
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
    // exp((z - m)/T) runs as exp2((z - m) * log2(e)/T) with that constant in fp32
    if (!(1.4426950408889634 / (double)temperature < (double)FLT_MAX)) return SV_ERR_INVALID_ARG;
    if (K > 0 && (!u_accept || !bt->draft)) return SV_ERR_INVALID_ARG;
  }
  if (need_draft) {
    if (bt->draft_ld < V || bt->draft_ld > (1ll << 40)) return SV_ERR_INVALID_ARG;
    if ((uintptr_t)bt->draft % es != 0) return SV_ERR_INVALID_ARG;
  }
  *zp = z;
  return SV_OK;
}

int32_t run(const sv_batch_t* bt, bool sample, float temperature, const uint8_t* gmask,
            const float* u_accept, const float* u_final, int32_t* acc_len, int32_t* out,
            float* p_out, float* q_out, float* resid_out, void* ws, size_t ws_bytes,
            void* stream, bool early_exit, int max_k) {
  // ---- host-side checks: nothing below touches the GPU until they pass
  Sizes z;
  const int32_t chk = host_checks(bt, sample, temperature, u_accept, u_final, acc_len, out,
                                  early_exit, max_k, &z);
  if (chk != SV_OK) return chk;
  if (!ws) return SV_ERR_WORKSPACE;
  if (ws_bytes < z.total) return SV_ERR_WORKSPACE;
  const long long B = bt->B, K = bt->K, V = bt->V;
  const int es = bt->dtype == SV_F32 ? 4 : 2;
  const bool need_draft = sample && K > 0;

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
    set_scale((double)temperature, &a.c, &a.c64);
    a.T64 = (double)temperature;
  } else {
    set_scale(1.0, &a.c, &a.c64);
    a.T64 = 1.0;
  }
  a.ws.hdr = reinterpret_cast<Header*>(wb + z.off_hdr);
  a.ws.req = reinterpret_cast<ReqInfo*>(wb + z.off_req);
  a.ws.rowdesc = reinterpret_cast<uint32_t*>(wb + z.off_rowdesc);
  a.ws.rowdesc_b = reinterpret_cast<uint32_t*>(wb + z.off_rowdesc_b);
  a.ws.stoch_list = reinterpret_cast<int*>(wb + z.off_resid);
  a.ws.pt = reinterpret_cast<Partial*>(wb + z.off_pt);
  a.ws.pd = reinterpret_cast<Partial*>(wb + z.off_pd);
  a.ws.rp = reinterpret_cast<double*>(wb + z.off_rp);
  a.ws.rows_r = reinterpret_cast<uint32_t*>(wb + z.off_rows_r);
  a.ws.res_r = reinterpret_cast<int*>(wb + z.off_res_r);
  a.ws.alive = nullptr;
  a.ws.alive_e = reinterpret_cast<AliveEntry*>(wb + z.off_alive);
  a.rowlist = a.ws.rowdesc;
  a.rowcount = &a.ws.hdr->n_rows;
  a.rowlist_b = a.ws.rowdesc_b;
  a.rowcount_b = &a.ws.hdr->n_rows_b;
  a.ee_round = -1;
  a.ee_lo = a.ee_hi = a.ee_nhi = 0;
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


}  // namespace

// ------------------------------------------------------------------ no-allocation entry point
// Workspace of spec_verify_sample_noalloc: one array of SPEC_VERIFY_NOALLOC_MAX_BYTES
// on every device the library runs on, held until the process ends.  In host
// code `scratch` only stands for the symbol; its device address on the current
// device comes from hipGetSymbolAddress, taken once per device and kept in
// g_scratch_addr, and only that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[SPEC_VERIFY_NOALLOC_MAX_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on device dev (the current device).
int32_t scratch_address(int dev, void** addr) {
  if (dev < 0 || dev >= kMaxDevices) return SV_ERR_HIP;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SV_ERR_HIP;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *addr = p;
  return SV_OK;
}
}  // namespace

extern "C" int32_t spec_verify_sample_noalloc(const sv_batch_t* batch, float temperature,
                                              const uint8_t* greedy_mask, const float* u_accept,
                                              const float* u_final, int32_t* accepted_len,
                                              int32_t* out_tokens, float* p_draft, float* q_draft,
                                              float* resid_mass, void* stream) {
  Sizes z;
  const int32_t chk = host_checks(batch, true, temperature, u_accept, u_final, accepted_len,
                                  out_tokens, false, 0, &z);
  if (chk != SV_OK) return chk;
  if (z.total > (size_t)SPEC_VERIFY_NOALLOC_MAX_BYTES) return SV_ERR_WORKSPACE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SV_ERR_HIP;
  void* ws = nullptr;
  const int32_t st = scratch_address(dev, &ws);
  if (st != SV_OK) return st;
  return run(batch, true, temperature, greedy_mask, u_accept, u_final, accepted_len, out_tokens,
             p_draft, q_draft, resid_mass, ws, (size_t)SPEC_VERIFY_NOALLOC_MAX_BYTES, stream, false, 0);
}


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





