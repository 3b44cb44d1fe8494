// fox_internal.h -- host-side launchers of the libfox kernels (not part of the public ABI).
// Each launcher assumes its arguments were validated by the C-ABI layer (fox_api.hip)
// and returns the HIP status of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fox {

// Inclusive prefix sums of `rows` independent rows of length n (fp64 accumulate).
hipError_t launch_logf_cumsum(const float* logf, float* c, int64_t rows, int n, hipStream_t stream);
// Suffix sums out_t = sum_{i>=t} (x_i - sub_i) of `rows` rows of length n (sub may be null; fp64
// accumulate).  x and sub are [rows, n]; out is [rows, n], or with token_major [rows / nh, n, nh].
hipError_t launch_suffix_sum(const float* x, const float* sub, float* out, int64_t rows, int n, int nh,
                             bool token_major, hipStream_t stream);

// FoX forward, causal (decoder mode) or over every key; is_bf16 selects the element type of
// q/k/v/o; d in {32,64,128}; token_major selects [B,N,H,d] tensors with [B,N,H] gates / lse /
// c instead of [B,H,N,d] and [B,H,N].
hipError_t launch_attn_fwd(const void* q, const void* k, const void* v, const float* logf, void* o, float* lse,
                           float* c, int64_t b, int64_t h, int n, int d, float scale, bool is_bf16, bool causal,
                           bool token_major, hipStream_t stream);

// Forward with gate-aware tile skipping (results equal to fp32 rounding); the workspace
// holds one float per (batch*head, 64-key tile).
size_t attn_fwd_pruned_workspace_bytes(int64_t bh, int n);
hipError_t launch_attn_fwd_pruned(const void* q, const void* k, const void* v, const float* logf, void* o,
                                  float* lse, float* c, float* workspace, int64_t bh, int n, int d, float scale,
                                  bool is_bf16, hipStream_t stream);

// Split-K decode: number of key splits used for these sizes, and the workspace it needs.
int decode_num_splits(int64_t sh, int l, int d);
size_t decode_workspace_bytes(int64_t sh, int l, int d);
// lens (device, one int per sequence, or nullptr): per-sequence cache lengths, clamped to
// [1, l]; nh = heads per sequence (sequence of (s, h) row sh is sh / nh).
hipError_t launch_attn_decode(const void* q, const void* kc, const void* vc, float* cc, const float* logf_new,
                              const int* lens, int nh, void* o, float* lse, float* workspace, int64_t sh, int l,
                              int d, float scale, bool is_bf16, hipStream_t stream);
// Device address of this device's fixed split-record array (FOX_DECODE_SCRATCH_BYTES), looked
// up on the first call per device (the current one).
hipError_t decode_scratch(float** out);
// The same step against paged caches: pools k/v [npages][nh][1 << page_shift][d], c [npages][nh][P],
// table [sequences][max_pages] (entries clamped to [0, npages)), lens required.
hipError_t launch_attn_decode_paged(const void* q, const void* kp, const void* vp, float* cp, const int* table,
                                    int max_pages, int page_shift, int npages, const float* logf_new, const int* lens,
                                    int nh, void* o, float* lse, float* ws, int64_t sh, int d, float scale,
                                    bool is_bf16, hipStream_t stream);

// The backward's gate terms (fox_bwd.hip): per row, block starts C_b of the prefix sums of log f
// (fp64, bwd_gate_blocks(n) per row, one per 32 positions up to n rounded up to 128) and, in the
// row-vector block [a | D | cl] of 3 * npad floats, a_i = (cq_i - lse_i) log2 e and cl_i = cq_i
// log2 e with cq_i = c_i - C_b(i), padded past n (a = -inf, D = 0, cl = +inf).  logf / lse are
// [rows, n], or with token_major [rows / nh, n, nh].
int bwd_gate_blocks(int n);
hipError_t launch_bwd_gate_rows(const float* logf, const float* lse, float* rowv, double* cb, int64_t rows, int n,
                                int npad, int nh, bool token_major, hipStream_t stream);

// Backward pass (bf16): dq, dk, dv and dlog f from q, k, v, the forward's o and lse, dO and the
// log gates; token_major as launch_attn_fwd.  Workspace: per-row vectors over n padded to 64,
// block starts of the gate sums (fp64), row and column sums of dS (attn_bwd_workspace_bytes).
size_t attn_bwd_workspace_bytes(int64_t bh, int n, int d);
// the staged backward (causal, bf16, d = 128): its workspace, the staged dS bytes of
// one head, and the launch
size_t attn_bwd_staged_workspace_bytes(int64_t bh, int n);
int64_t attn_bwd_staged_head_bytes(int n);
hipError_t launch_attn_bwd_staged(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                  const float* lse, const float* logf, void* dq, void* dk, void* dv, float* dlogf,
                                  void* workspace, int64_t b, int64_t h, int n, float scale, bool token_major,
                                  hipStream_t stream);
hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, const float* logf, void* dq, void* dk, void* dv, float* dlogf,
                           void* workspace, int64_t b, int64_t h, int n, int d, float scale, bool causal,
                           bool token_major, hipStream_t stream);
// The same on fp32 tensors (fp32 throughout; same workspace size and layouts).
hipError_t launch_attn_bwd_f32(const float* q, const float* k, const float* v, const float* o, const float* dout,
                               const float* lse, const float* logf, float* dq, float* dk, float* dv, float* dlogf,
                               void* workspace, int64_t b, int64_t h, int n, int d, float scale, bool causal,
                               bool token_major, hipStream_t stream);
// Workspace carve-up shared by both backward paths.
struct BwdWorkspace {
  float* rowv;  // [bh][3][npad]
  double* cb;   // [bh][bwd_gate_blocks(n)]
  float* rsum;  // [bh][n]
  float* csum;  // [bh][n]
  float* corr;  // [bh][n]: the fp32 path's lse normalisation (unmasked mode)
};
BwdWorkspace bwd_workspace(void* ws, int64_t bh, int n, int npad);

}  // namespace fox
