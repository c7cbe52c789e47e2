// probe.hip - plain streaming read with the access pattern of the row-statistics
// kernel (diagnostic; implements spec_verify_read_probe of include/spec_verify.h).
//
// A persistent grid of one wavefront per 32 KiB unit, as many resident
// workgroups per CU as the occupancy calculator allows (at most 8), reads the
// buffer once with 16-byte nontemporal loads, four in flight per lane, and
// does nothing with the data but fold it into one xor per wavefront (so the
// loads cannot be dropped).  Its bandwidth is the
// ceiling the streaming kernels are measured against.  The sink receives a
// store only if a wavefront's xor equals one fixed value; it needs 64 words.
#include "sv_common.hpp"

namespace {

constexpr int kProbeUnroll = 4;

__global__ __launch_bounds__(kBlock) void k_read_probe(const uint4* src, long long n16,
                                                       unsigned int* sink) {
  const int lane = threadIdx.x & (kWave - 1);
  const int gw = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int W = gridDim.x * kWavesPerBlock;
  constexpr long long kUnit16 = kSegBytes / 16;       // 16-byte chunks per unit
  const long long n_units = (n16 + kUnit16 - 1) / kUnit16;
  unsigned int acc = 0;
  for (long long u = gw; u < n_units; u += W) {
    const long long c0 = u * kUnit16;
    const long long c1 = c0 + kUnit16 < n16 ? c0 + kUnit16 : n16;
    long long c = c0 + lane;
    for (; c + (kProbeUnroll - 1) * kWave < c1; c += kProbeUnroll * kWave) {
      u32x4 r[kProbeUnroll];
#pragma unroll
      for (int j = 0; j < kProbeUnroll; ++j)
        r[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + c + j * kWave));
#pragma unroll
      for (int j = 0; j < kProbeUnroll; ++j) acc ^= r[j].x ^ r[j].y ^ r[j].z ^ r[j].w;
    }
    for (; c < c1; c += kWave) {
      const u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + c));
      acc ^= r.x ^ r.y ^ r.z ^ r.w;
    }
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  if (acc == 0x9e3779b9u) sink[lane] = acc;   // (data-dependent store: keeps the loads alive)
}

std::atomic<int> g_occ_probe[64];

}  // namespace

extern "C" int32_t spec_verify_read_probe(const void* src, size_t bytes, uint32_t* sink,
                                          void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 || (uintptr_t)src % 16 != 0)
    return SV_ERR_INVALID_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SV_ERR_HIP;
  const long long n16 = (long long)(bytes / 16);
  const long long units = (n16 * 16 + kSegBytes - 1) / kSegBytes;
  const long long cap = (long long)cu_count(dev) * resident_blocks(g_occ_probe, k_read_probe, dev);
  const int grid = (int)std::max(1ll, std::min(cap, (units + kWavesPerBlock - 1) / kWavesPerBlock));
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (g_ev_begin && g_ev_end) (void)hipEventRecord((hipEvent_t)g_ev_begin, st);
  k_read_probe<<<grid, kBlock, 0, st>>>(static_cast<const uint4*>(src), n16,
                                         reinterpret_cast<unsigned int*>(sink));
  if (g_ev_begin && g_ev_end) (void)hipEventRecord((hipEvent_t)g_ev_end, st);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_HIP;
}
