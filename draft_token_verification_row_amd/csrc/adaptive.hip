// adaptive.hip - confidence-driven verification length with compaction of
// the kept windows, and the row gather that moves the kept draft rows.
#include "sv_common.hpp"

namespace {

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

#ifndef SV_GATHER_UNROLL
#define SV_GATHER_UNROLL 16
#endif
constexpr int kGatherUnroll = SV_GATHER_UNROLL;

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
      // kGatherUnroll 16-byte loads in flight per lane, then their stores (16
      // divides a 32 KiB piece: 32 chunks per lane, two steps, no tail loop)
      constexpr long long kStep = (long long)kWave * 16;
      long long o = p0 + (long long)lane * 16;
      for (; o + (kGatherUnroll - 1) * kStep + 16 <= p1; o += kGatherUnroll * kStep) {
        u32x4 v[kGatherUnroll];
#pragma unroll
        for (int j = 0; j < kGatherUnroll; ++j)
          v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(s + o + j * kStep));
#pragma unroll
        for (int j = 0; j < kGatherUnroll; ++j)
          __builtin_nontemporal_store(v[j], reinterpret_cast<u32x4*>(d + o + j * kStep));
      }
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

}  // namespace

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
