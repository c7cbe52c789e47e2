// accept_stats.hip - acceptance statistics of verification outcomes.
#include "sv_common.hpp"

namespace {

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

}  // namespace

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
