// fox_decode.hip -- K3/K4: causal FoX decode step against a KV cache (split-K, HBM-bound).
//
// For each (sequence, head) the new query attends to all L cache slots:
//   s_j = scale * q.k_j + (c_new - c_j),   c_new = c_{L-2} + log f_new,   c_{L-1} = c_new,
// which is the last row of the forward definition (FoX module page,
// ForgettingAttention.forward; foxwindow README, opening paragraph).  The pages
// define no cache; the slot convention is documented in include/fox.h.
//
// K3 (decode_split_kernel): the L keys are cut into `nsplit` chunks; one 256-thread
//   workgroup streams one chunk of one (sequence, head) exactly once.  A key row of
//   d elements is spread over G lanes, 16 bytes each (bf16 d=128: 16 lanes), so one
//   wave64 load instruction covers 64/G whole keys and every load is a full, aligned
//   16-byte access; kDecU steps are unrolled so 2*kDecU loads per lane are in flight.
//   Dot products run on VALU in fp32 with a DPP reduction inside the G-lane group;
//   the gate bias is (c_{L-2} - c_j) + log f_new, which is exact in fp32 for nearby j.
//   The chunk is walked from its last key backwards (largest bias first) with the
//   same lazy base-2 online softmax as the forward kernel.  Each workgroup reduces its
//   (max, sum, acc[d]) over lane groups and waves and writes one partial record.
// K4 (decode_combine_kernel): merges the records of one (sequence, head) by the
//   log-sum-exp rule, writes O, lse and the new prefix sum into cache slot L-1.
//
// Ragged caches: with `lens` given, sequence s uses only its first lens[s] slots (clamped to
// [1, L]) of caches allocated for L, and its new token sits at slot lens[s]-1.  Its slots are
// shared evenly by its nsplit workgroups; a split left without slots writes an empty record.
// The split workgroups take the sequences in decreasing order of length.
// Paged caches (PAGED): logical slot j of sequence s is row j & (P-1) of physical page
// table[s][j >> log2 P] in pools [pages][heads][P][d] (c: [pages][heads][P]); the capacity L is
// max_pages * P.  Everything else is the ragged step.
#include <math.h>

#include <algorithm>
#include <atomic>

#include "../../include/fox.h"
#include "fox_device.h"
#include "fox_internal.h"

namespace fox {
namespace {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kDecU = 4;
constexpr int kRankSeqs = 1024;  // ragged caches: sequences ordered by length on the device up to this many
constexpr float kTau = 8.0f;
constexpr float kNegInf = -INFINITY;

template <typename T, int D>
struct DecCfg {
  static constexpr int EPL = 16 / (int)sizeof(T);  // elements per 16-byte load
  static constexpr int G = D / EPL;                // lanes per key
  static constexpr int KPW = 64 / G;               // keys per wave per step
  static constexpr int KPB = kDecWaves * KPW;      // keys per workgroup per step
  static constexpr int REC = D + 2;                // floats per partial record: m, l, acc[D]
};

template <typename T>
struct Vec16;
template <>
struct Vec16<bf16> {
  u32x4 w;
  __device__ __forceinline__ void load(const bf16* p) { w = *reinterpret_cast<const u32x4*>(p); }
  __device__ __forceinline__ void zero() { w = u32x4{0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ float get(int e) const { return (e & 1) ? bf16hi(w[e >> 1]) : bf16lo(w[e >> 1]); }
};
template <>
struct Vec16<float> {
  f32x4 w;
  __device__ __forceinline__ void load(const float* p) { w = *reinterpret_cast<const f32x4*>(p); }
  __device__ __forceinline__ void zero() { w = f32x4{}; }
  __device__ __forceinline__ float get(int e) const { return w[e]; }
};

__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }

// Where a (sequence, head)'s logical cache slot lives: the row index into the K / V caches (times d
// for the element offset) and the index into the c cache.
struct PageMap {
  const int* table;  // [sequences][max_pages] physical page numbers, or null (contiguous caches)
  int max_pages;
  int shift;   // log2 of the page size
  int npages;  // pages in the pools (table entries are clamped to [0, npages))
};
template <bool PAGED>
__device__ __forceinline__ size_t cache_row(const PageMap& pm, int sh, int nh, int Lcap, int slot) {
  if constexpr (PAGED) {
    const int s = sh / nh, h = sh - s * nh;
    int pg = pm.table[(size_t)s * pm.max_pages + (slot >> pm.shift)];
    pg = min(max(pg, 0), pm.npages - 1);
    return (((size_t)pg * nh + h) << pm.shift) + (size_t)(slot & ((1 << pm.shift) - 1));
  } else {
    return (size_t)sh * Lcap + slot;
  }
}

// Merge running softmax state (m, l, acc) with another in base 2; either may be empty (m = -inf).
template <int N>
__device__ __forceinline__ void merge_state(float& m, float& l, float (&acc)[N], float mo, float lo,
                                            const float (&acco)[N]) {
  const float mn = fmaxf(m, mo);
  const float a = (m == kNegInf) ? 0.0f : exp2_hw(m - mn);
  const float b = (mo == kNegInf) ? 0.0f : exp2_hw(mo - mn);
  l = l * a + lo * b;
#pragma unroll
  for (int e = 0; e < N; ++e) acc[e] = acc[e] * a + acco[e] * b;
  m = mn;
}

template <typename T, int D, bool PAGED>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(const T* __restrict__ q, const T* __restrict__ kc,
                                                                  const T* __restrict__ vc,
                                                                  const float* __restrict__ cc,
                                                                  const float* __restrict__ logf_new,
                                                                  float* __restrict__ part, int Lcap,
                                                                  const int* __restrict__ lens, int nh, int nsplit,
                                                                  int chunk, float scale_log2, PageMap pm) {
  using C = DecCfg<T, D>;
  constexpr int EPL = C::EPL, G = C::G, KPW = C::KPW, KPB = C::KPB;
  __shared__ float s_m[kDecWaves], s_l[kDecWaves];
  __shared__ float s_acc[kDecWaves][D];

  // Ragged caches: the workgroups take the sequences longest first (decreasing length, ties by
  // index), so that no long sequence's splits start last and hold up the end of the grid.  Each
  // (sequence, head, split) computes what it does in plain order; only the dispatch order changes.
  int wg = blockIdx.x;
  if (lens) {
    const int per = nh * nsplit;  // workgroups per sequence
    const int nseq = (int)(gridDim.x / (unsigned)per);
    if (nseq <= kRankSeqs) {
      __shared__ int s_len[kRankSeqs];
      __shared__ int s_pick;
      for (int t = threadIdx.x; t < nseq; t += kDecThreads) s_len[t] = min(max(lens[t], 1), Lcap);
      __syncthreads();
      const int r = wg / per;  // this workgroup serves the sequence of rank r
      for (int t = threadIdx.x; t < nseq; t += kDecThreads) {
        const int lt = s_len[t];
        int rank = 0;
        for (int u = 0; u < nseq; ++u) rank += (s_len[u] > lt) || (s_len[u] == lt && u < t);
        if (rank == r) s_pick = t;
      }
      __syncthreads();
      wg = s_pick * per + (wg - r * per);
    }
  }
  const int sh = wg / nsplit, split = wg - sh * nsplit;
  const int L = lens ? min(max(lens[sh / nh], 1), Lcap) : Lcap;  // this sequence's slots
  // a sequence's slots are shared evenly by its nsplit workgroups (with every length at the
  // capacity this is the fixed chunk), so no workgroup of a short sequence sits idle
  const int ck = lens ? (L + nsplit - 1) / nsplit : chunk;
  const int start = split * ck;
  const int end = min(L, start + ck);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane % G;
  const int slot = lane / G + KPW * wave;
  const T* kp = kc + g * EPL;
  const T* vp = vc + g * EPL;

  float qv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) qv[e] = to_f32(q[(size_t)sh * D + g * EPL + e]) * scale_log2;
  const float lnew = logf_new[sh];
  const float cprev = (L >= 2) ? cc[cache_row<PAGED>(pm, sh, nh, Lcap, L - 2)] : 0.0f;

  float m = kNegInf, l = 0.0f, acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;

  const int nsteps = end > start ? (end - start + KPB - 1) / KPB : 0;
  for (int s0 = nsteps - 1; s0 >= 0; s0 -= kDecU) {
    Vec16<T> kr[kDecU], vr[kDecU];
    float cj[kDecU];
    int key[kDecU];
#pragma unroll
    for (int u = 0; u < kDecU; ++u) {
      key[u] = start + (s0 - u) * KPB + slot;
      const bool ok = (s0 - u >= 0) && key[u] < end;
      if (ok) {
        const size_t row = cache_row<PAGED>(pm, sh, nh, Lcap, key[u]);
        kr[u].load(kp + row * D);
        vr[u].load(vp + row * D);
        cj[u] = (key[u] < L - 1) ? cc[row] : cprev;
      } else {
        kr[u].zero();
        vr[u].zero();
        cj[u] = cprev;
        key[u] = -1;
      }
    }
    float s[kDecU];
    float mx = kNegInf;
#pragma unroll
    for (int u = 0; u < kDecU; ++u) {
      float dot = 0.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) dot = fmaf(qv[e], kr[u].get(e), dot);
      dot = group_sum<G>(dot);
      // bias c_new - c_j = (c_{L-2} - c_j) + log f_new for j <= L-2, and 0 for j = L-1
      const float bias = (key[u] == L - 1) ? 0.0f : ((cprev - cj[u]) + lnew) * kLog2e;
      s[u] = (key[u] >= 0) ? dot + bias : kNegInf;
      mx = fmaxf(mx, s[u]);
    }
    const float mcand = fmaxf(m, mx);
    const bool need = mcand > m + kTau;
    if (wave_any(need)) {
      const float mn = need ? mcand : m;
      const float alpha = (m == kNegInf) ? 0.0f : exp2_hw(m - mn);
      l *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] *= alpha;
      m = mn;
    }
    const float msub = (m == kNegInf) ? 0.0f : m;
#pragma unroll
    for (int u = 0; u < kDecU; ++u) {
      const float p = exp2_hw(s[u] - msub);  // exactly 0 for padding keys (s = -inf)
      l += p;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = fmaf(p, vr[u].get(e), acc[e]);
    }
  }

  // lane groups of one wave hold the same dims for different keys: merge them
#pragma unroll
  for (int off = G; off < 64; off <<= 1) {
    float acco[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acco[e] = __shfl_xor(acc[e], off);
    const float mo = __shfl_xor(m, off), lo = __shfl_xor(l, off);
    merge_state(m, l, acc, mo, lo, acco);
  }
  if (lane < G) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) s_acc[wave][g * EPL + e] = acc[e];
    if (lane == 0) {
      s_m[wave] = m;
      s_l[wave] = l;
    }
  }
  __syncthreads();
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, s_m[w]);
  float* rec = part + (size_t)wg * C::REC;
  for (int t = tid; t < D; t += kDecThreads) {
    float a = 0.0f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w)
      if (s_m[w] != kNegInf) a += s_acc[w][t] * exp2_hw(s_m[w] - M);
    rec[2 + t] = a;
  }
  if (tid == 0) {
    float lt = 0.0f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w)
      if (s_m[w] != kNegInf) lt += s_l[w] * exp2_hw(s_m[w] - M);
    rec[0] = M;
    rec[1] = lt;
  }
}

template <typename T>
__device__ __forceinline__ void store_out(T* p, float x);
template <>
__device__ __forceinline__ void store_out<bf16>(bf16* p, float x) {
  *p = (bf16)x;
}
template <>
__device__ __forceinline__ void store_out<float>(float* p, float x) {
  *p = x;
}

template <typename T, int D, bool PAGED>
__global__ __launch_bounds__(64) void decode_combine_kernel(const float* __restrict__ part, T* __restrict__ o,
                                                           float* __restrict__ lse, float* __restrict__ cc,
                                                           const float* __restrict__ logf_new, int Lcap,
                                                           const int* __restrict__ lens, int nh, int nsplit,
                                                           PageMap pm) {
  constexpr int REC = D + 2;
  const int sh = blockIdx.x;
  const int lane = threadIdx.x;
  const float* recs = part + (size_t)sh * nsplit * REC;
  float M = kNegInf;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, recs[(size_t)s * REC]);
  float lt = 0.0f;
  constexpr int PER = (D + 63) / 64;
  float a[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) a[i] = 0.0f;
  for (int s = 0; s < nsplit; ++s) {
    const float* r = recs + (size_t)s * REC;
    const float ms = r[0];
    if (ms == kNegInf) continue;
    const float w = exp2_hw(ms - M);
    lt += r[1] * w;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int dd = lane + 64 * i;
      if (dd < D) a[i] += r[2 + dd] * w;
    }
  }
  const float inv = 1.0f / lt;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int dd = lane + 64 * i;
    if (dd < D) store_out<T>(o + (size_t)sh * D + dd, a[i] * inv);
  }
  if (lane == 0) {
    if (lse) lse[sh] = (float)(((double)M + (double)log2f(lt)) * kLn2d);
    const int L = lens ? min(max(lens[sh / nh], 1), Lcap) : Lcap;
    const float cprev = (L >= 2) ? cc[cache_row<PAGED>(pm, sh, nh, Lcap, L - 2)] : 0.0f;
    cc[cache_row<PAGED>(pm, sh, nh, Lcap, L - 1)] = cprev + logf_new[sh];
  }
}

template <typename T, int D, bool PAGED>
hipError_t launch_decode_p(const void* q, const void* kc, const void* vc, float* cc, const float* logf_new,
                           const int* lens, int nh, void* o, float* lse, float* ws, int64_t sh, int l, float scale,
                           const PageMap& pm, hipStream_t stream) {
  const int nsplit = decode_num_splits(sh, l, D);
  const int chunk = (l + nsplit - 1) / nsplit;
  const float scale_log2 = (float)((double)scale * kLog2ed);
  hipLaunchKernelGGL((decode_split_kernel<T, D, PAGED>), dim3((unsigned)(sh * nsplit)), dim3(kDecThreads), 0, stream,
                     (const T*)q, (const T*)kc, (const T*)vc, (const float*)cc, logf_new, ws, l, lens, nh, nsplit,
                     chunk, scale_log2, pm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T, D, PAGED>), dim3((unsigned)sh), dim3(64), 0, stream, (const float*)ws,
                     (T*)o, lse, cc, logf_new, l, lens, nh, nsplit, pm);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_decode_t(const void* q, const void* kc, const void* vc, float* cc, const float* logf_new,
                           const int* lens, int nh, void* o, float* lse, float* ws, int64_t sh, int l, float scale,
                           const PageMap& pm, hipStream_t stream) {
  if (pm.table) return launch_decode_p<T, D, true>(q, kc, vc, cc, logf_new, lens, nh, o, lse, ws, sh, l, scale, pm, stream);
  return launch_decode_p<T, D, false>(q, kc, vc, cc, logf_new, lens, nh, o, lse, ws, sh, l, scale, pm, stream);
}

}  // namespace

int decode_num_splits(int64_t sh, int l, int d) {
  (void)d;
  // Enough workgroups to cover the 256 CUs many times over (>= 8192 in total), but
  // never fewer than 256 keys per split, and no empty split.
  const int64_t want = std::max<int64_t>(1, (8192 + sh - 1) / sh);
  const int64_t most = std::max(1, l / 256);
  const int ns = (int)std::min(want, most);
  const int chunk = (l + ns - 1) / ns;
  return (l + chunk - 1) / chunk;
}

size_t decode_workspace_bytes(int64_t sh, int l, int d) {
  return (size_t)sh * (size_t)decode_num_splits(sh, l, d) * (size_t)(d + 2) * sizeof(float);
}

namespace {

hipError_t launch_decode_any(const void* q, const void* kc, const void* vc, float* cc, const float* logf_new,
                             const int* lens, int nh, void* o, float* lse, float* ws, int64_t sh, int l, int d,
                             float scale, bool is_bf16, const PageMap& pm, hipStream_t stream) {
  if (is_bf16) {
    switch (d) {
      case 32: return launch_decode_t<bf16, 32>(q, kc, vc, cc, logf_new, lens, nh, o, lse, ws, sh, l, scale, pm, stream);
      case 64: return launch_decode_t<bf16, 64>(q, kc, vc, cc, logf_new, lens, nh, o, lse, ws, sh, l, scale, pm, stream);
      case 128:
        return launch_decode_t<bf16, 128>(q, kc, vc, cc, logf_new, lens, nh, o, lse, ws, sh, l, scale, pm, stream);
    }
  } else {
    switch (d) {
      case 32: return launch_decode_t<float, 32>(q, kc, vc, cc, logf_new, lens, nh, o, lse, ws, sh, l, scale, pm, stream);
      case 64: return launch_decode_t<float, 64>(q, kc, vc, cc, logf_new, lens, nh, o, lse, ws, sh, l, scale, pm, stream);
      case 128:
        return launch_decode_t<float, 128>(q, kc, vc, cc, logf_new, lens, nh, o, lse, ws, sh, l, scale, pm, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attn_decode(const void* q, const void* kc, const void* vc, float* cc, const float* logf_new,
                              const int* lens, int nh, void* o, float* lse, float* ws, int64_t sh, int l, int d,
                              float scale, bool is_bf16, hipStream_t stream) {
  const PageMap pm{nullptr, 0, 0, 0};
  return launch_decode_any(q, kc, vc, cc, logf_new, lens, nh, o, lse, ws, sh, l, d, scale, is_bf16, pm, stream);
}

// Split records of fox_attn_decode_noalloc: a fixed device array instead of a caller workspace,
// FOX_DECODE_SCRATCH_BYTES per device for the life of the process.  Host code never uses its
// name as an address (on the host it stands for the variable, not its device location): the
// device address comes from hipGetSymbolAddress, looked up once per device with that device
// current, and is what the kernels receive.  The kernels write every record before the combine
// reads it, so nothing needs clearing between calls; calls that overlap on one device race on it.
static __device__ __align__(256) float scratch[FOX_DECODE_SCRATCH_BYTES / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<float*> g_scratch[kMaxDevices];  // this device's address of `scratch`, once looked up
}  // namespace

hipError_t decode_scratch(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  float* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!a) return hipErrorInvalidSymbol;
    p = static_cast<float*>(a);
    g_scratch[dev].store(p, std::memory_order_release);  // same value from any racing thread
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_attn_decode_paged(const void* q, const void* kp, const void* vp, float* cp, const int* table,
                                    int max_pages, int page_shift, int npages, const float* logf_new, const int* lens,
                                    int nh, void* o, float* lse, float* ws, int64_t sh, int d, float scale,
                                    bool is_bf16, hipStream_t stream) {
  const PageMap pm{table, max_pages, page_shift, npages};
  return launch_decode_any(q, kp, vp, cp, logf_new, lens, nh, o, lse, ws, sh, max_pages << page_shift, d, scale,
                           is_bf16, pm, stream);
}

}  // namespace fox
