// fox_scan.hip -- K1: inclusive prefix sum of log forget gates, c_i = sum_{t<=i} log f_t.
//
// FoX module page, ForgettingAttention.forward: the cumulative sum of log f
// along the sequence axis.  One 256-thread workgroup per (batch, head) row walks
// the row in chunks of 1024 elements: each thread sums 4 consecutive gates, a
// wave64 DPP scan and a 4-entry LDS scan give the chunk prefix, and a carry
// links the chunks; the next chunk's loads are issued before the current chunk's
// scan, and the wave totals alternate between two LDS slots (one barrier per
// chunk).  Accumulation is fp64 (|c| reaches ~10^3 at 8k tokens, where an fp32
// running sum would drift); each c is rounded to fp32 once.
#include "fox_device.h"
#include "fox_internal.h"

namespace fox {
namespace {

constexpr int kScanThreads = 256;
constexpr int kScanPerThread = 4;
constexpr int kScanChunk = kScanThreads * kScanPerThread;

// Where output row `row` (= batch * nh + head) lives: element t at (row / nh) bs + (row % nh) hs + t es.
struct OutRows {
  int nh;
  int64_t bs, hs;
  int es;
};

// REV: the suffix sums out_t = sum_{i>=t} (in_i - sub_i) instead (the same scan over the reversed
// row; sub may be null).  Inputs are [rows, n]; the output rows are placed by `om`.
template <bool REV>
__global__ __launch_bounds__(kScanThreads) void logf_cumsum_kernel(const float* __restrict__ logf,
                                                                   const float* __restrict__ sub,
                                                                   float* __restrict__ c, int n, OutRows om) {
  __shared__ double wave_tot[2][kScanThreads / 64];  // per chunk parity: one barrier per chunk
  const size_t row = blockIdx.x;
  const float* src = logf + row * (size_t)n;
  const float* sb = sub ? sub + row * (size_t)n : nullptr;
  float* dst = c + (int64_t)(row / om.nh) * om.bs + (int64_t)(row % om.nh) * om.hs;
  const int64_t es = om.es;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // the loads of chunk `base` (element i0 + e of the scan order, 0 past n)
  auto load = [&](int base, float (&xv)[kScanPerThread], float (&sv)[kScanPerThread]) {
    const int i0 = base + tid * kScanPerThread;
#pragma unroll
    for (int e = 0; e < kScanPerThread; ++e) {
      const int j = REV ? n - 1 - (i0 + e) : i0 + e;
      const bool in = i0 + e < n;
      xv[e] = in ? src[j] : 0.0f;
      sv[e] = in && sb ? sb[j] : 0.0f;
    }
  };
  float xa[kScanPerThread], sa[kScanPerThread];
  load(0, xa, sa);
  double carry = 0.0;
  for (int base = 0, it = 0; base < n; base += kScanChunk, ++it) {
    double x[kScanPerThread];
#pragma unroll
    for (int e = 0; e < kScanPerThread; ++e) x[e] = (double)xa[e] - (double)sa[e];
    if (base + kScanChunk < n) load(base + kScanChunk, xa, sa);  // the next chunk's loads in flight
#pragma unroll
    for (int e = 1; e < kScanPerThread; ++e) x[e] += x[e - 1];
    const double t = wave_incl_scan(x[kScanPerThread - 1]);  // over this wave's threads
    const double excl = wave_shr1(t);
    if (lane == 63) wave_tot[it & 1][wave] = t;
    __syncthreads();
    double before = carry, chunk = 0.0;
#pragma unroll
    for (int w = 0; w < kScanThreads / 64; ++w) {
      if (w < wave) before += wave_tot[it & 1][w];
      chunk += wave_tot[it & 1][w];
    }
    const double pre = before + excl;
    const int i0 = base + tid * kScanPerThread;
#pragma unroll
    for (int e = 0; e < kScanPerThread; ++e)
      if (i0 + e < n) dst[(REV ? n - 1 - (i0 + e) : i0 + e) * es] = (float)(pre + x[e]);
    carry += chunk;
  }
}

}  // namespace

hipError_t launch_logf_cumsum(const float* logf, float* c, int64_t rows, int n, hipStream_t stream) {
  hipLaunchKernelGGL(logf_cumsum_kernel<false>, dim3((unsigned)rows), dim3(kScanThreads), 0, stream, logf,
                     (const float*)nullptr, c, n, OutRows{1, (int64_t)n, 0, 1});
  return hipGetLastError();
}

hipError_t launch_suffix_sum(const float* x, const float* sub, float* out, int64_t rows, int n, int nh,
                             bool token_major, hipStream_t stream) {
  const OutRows om = token_major ? OutRows{nh, (int64_t)n * nh, 1, nh} : OutRows{1, (int64_t)n, 0, 1};
  hipLaunchKernelGGL(logf_cumsum_kernel<true>, dim3((unsigned)rows), dim3(kScanThreads), 0, stream, x, sub, out, n,
                     om);
  return hipGetLastError();
}

}  // namespace fox
