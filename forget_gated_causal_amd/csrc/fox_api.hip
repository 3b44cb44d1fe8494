// fox_api.hip -- the C ABI of libfox (declared in include/fox.h): argument
// validation on the host, then kernel launches on the caller's stream.
// Nothing is launched when validation fails; no allocation, no synchronisation.
#include <math.h>
#include <stdint.h>

#include "../../include/fox.h"
#include "fox_internal.h"

namespace {

constexpr int64_t kI32Max = 2147483647;
constexpr int64_t kMaxGridY = 65535;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// [p, p + bytes) and [q, q + qbytes) overlap
bool overlap(const void* p, size_t bytes, const void* q, size_t qbytes) {
  if (!p || !q) return false;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + qbytes && b < a + bytes;
}

bool head_dim_ok(int64_t d) { return d == 32 || d == 64 || d == 128; }
bool dtype_ok(fox_dtype_t t) { return t == FOX_F32 || t == FOX_BF16; }
size_t elem_bytes(fox_dtype_t t) { return t == FOX_BF16 ? 2 : 4; }
bool scale_ok(float s) { return isfinite(s) && s > 0.0f; }

fox_status_t from_hip(hipError_t e) { return e == hipSuccess ? FOX_OK : FOX_ERR_HIP; }

}  // namespace

extern "C" {

const char* fox_status_string(fox_status_t status) {
  switch (status) {
    case FOX_OK: return "ok";
    case FOX_ERR_INVALID_ARG: return "invalid argument (null pointer, bad size, bad scale, misaligned or aliased buffer)";
    case FOX_ERR_UNSUPPORTED: return "unsupported head dim (need 32, 64 or 128) or dtype";
    case FOX_ERR_WORKSPACE: return "decode workspace missing, misaligned or too small";
    case FOX_ERR_HIP: return "HIP runtime error at kernel launch";
    case FOX_ERR_SCRATCH: return "sizes need more split-record space than the fixed decode scratch holds";
  }
  return "unknown status";
}

fox_status_t fox_logf_cumsum(const float* logf, float* c, int64_t rows, int64_t n, hipStream_t stream) {
  if (!logf || !c) return FOX_ERR_INVALID_ARG;
  if (rows <= 0 || n <= 0 || n > FOX_MAX_SEQ || rows > kI32Max) return FOX_ERR_INVALID_ARG;
  if (!aligned(logf, 4) || !aligned(c, 4)) return FOX_ERR_INVALID_ARG;
  const size_t bytes = (size_t)rows * (size_t)n * sizeof(float);
  if (overlap(logf, bytes, c, bytes)) return FOX_ERR_INVALID_ARG;
  return from_hip(fox::launch_logf_cumsum(logf, c, rows, (int)n, stream));
}

// Validation shared by the forward entry points.
static fox_status_t fwd_args(const void* q, const void* k, const void* v, const float* logf, void* o, float* lse,
                             float* c, int64_t b, int64_t h, int64_t n, int64_t d, float scale, fox_dtype_t dtype) {
  if (!q || !k || !v || !logf || !o) return FOX_ERR_INVALID_ARG;
  if (b <= 0 || h <= 0 || n <= 0 || d <= 0 || n > FOX_MAX_SEQ) return FOX_ERR_INVALID_ARG;
  if (b > kI32Max / h) return FOX_ERR_INVALID_ARG;
  if (!dtype_ok(dtype) || !head_dim_ok(d)) return FOX_ERR_UNSUPPORTED;
  if (!scale_ok(scale)) return FOX_ERR_INVALID_ARG;
  if ((n + 127) / 128 > kMaxGridY) return FOX_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return FOX_ERR_INVALID_ARG;
  if (!aligned(logf, 4) || !aligned(lse, 4) || !aligned(c, 4)) return FOX_ERR_INVALID_ARG;
  const int64_t bh = b * h;
  const size_t tbytes = (size_t)bh * (size_t)n * (size_t)d * elem_bytes(dtype);
  const size_t vbytes = (size_t)bh * (size_t)n * sizeof(float);
  if (overlap(o, tbytes, q, tbytes) || overlap(o, tbytes, k, tbytes) || overlap(o, tbytes, v, tbytes) ||
      overlap(o, tbytes, logf, vbytes) || overlap(lse, vbytes, logf, vbytes) || overlap(c, vbytes, logf, vbytes) ||
      overlap(lse, vbytes, c, vbytes) || overlap(lse, vbytes, o, tbytes) || overlap(c, vbytes, o, tbytes) ||
      overlap(lse, vbytes, q, tbytes) || overlap(lse, vbytes, k, tbytes) || overlap(lse, vbytes, v, tbytes) ||
      overlap(c, vbytes, q, tbytes) || overlap(c, vbytes, k, tbytes) || overlap(c, vbytes, v, tbytes))
    return FOX_ERR_INVALID_ARG;
  return FOX_OK;
}

fox_status_t fox_attn_fwd_ex(const void* q, const void* k, const void* v, const float* logf, void* o, float* lse,
                             float* c, int64_t b, int64_t h, int64_t n, int64_t d, float scale, fox_dtype_t dtype,
                             int causal, fox_layout_t layout, hipStream_t stream) {
  const fox_status_t st = fwd_args(q, k, v, logf, o, lse, c, b, h, n, d, scale, dtype);
  if (st != FOX_OK) return st;
  if (layout != FOX_HEAD_MAJOR && layout != FOX_TOKEN_MAJOR) return FOX_ERR_UNSUPPORTED;
  // token-major: one head's rows span (n-1)*h*d + d elements, addressed with 32-bit byte offsets
  if (layout == FOX_TOKEN_MAJOR && (n + 64) * h * d * (int64_t)elem_bytes(dtype) > kI32Max) return FOX_ERR_UNSUPPORTED;
  return from_hip(fox::launch_attn_fwd(q, k, v, logf, o, lse, c, b, h, (int)n, (int)d, scale, dtype == FOX_BF16,
                                       causal != 0, layout == FOX_TOKEN_MAJOR, stream));
}

fox_status_t fox_attn_fwd(const void* q, const void* k, const void* v, const float* logf, void* o, float* lse,
                          float* c, int64_t b, int64_t h, int64_t n, int64_t d, float scale, fox_dtype_t dtype,
                          hipStream_t stream) {
  return fox_attn_fwd_ex(q, k, v, logf, o, lse, c, b, h, n, d, scale, dtype, 1, FOX_HEAD_MAJOR, stream);
}

fox_status_t fox_attn_fwd_noncausal(const void* q, const void* k, const void* v, const float* logf, void* o,
                                    float* lse, float* c, int64_t b, int64_t h, int64_t n, int64_t d, float scale,
                                    fox_dtype_t dtype, hipStream_t stream) {
  return fox_attn_fwd_ex(q, k, v, logf, o, lse, c, b, h, n, d, scale, dtype, 0, FOX_HEAD_MAJOR, stream);
}

size_t fox_attn_fwd_pruned_workspace_bytes(int64_t b, int64_t h, int64_t n, int64_t d) {
  if (b <= 0 || h <= 0 || n <= 0 || n > FOX_MAX_SEQ || !head_dim_ok(d) || b > kI32Max / h) return 0;
  return fox::attn_fwd_pruned_workspace_bytes(b * h, (int)n);
}

fox_status_t fox_attn_fwd_pruned(const void* q, const void* k, const void* v, const float* logf, void* o,
                                 float* lse, float* c, void* workspace, size_t workspace_bytes, int64_t b, int64_t h,
                                 int64_t n, int64_t d, float scale, fox_dtype_t dtype, hipStream_t stream) {
  const fox_status_t st = fwd_args(q, k, v, logf, o, lse, c, b, h, n, d, scale, dtype);
  if (st != FOX_OK) return st;
  const int64_t bh = b * h;
  const size_t need = fox::attn_fwd_pruned_workspace_bytes(bh, (int)n);
  if (!workspace || !aligned(workspace, 16) || workspace_bytes < need) return FOX_ERR_WORKSPACE;
  const size_t tbytes = (size_t)bh * (size_t)n * (size_t)d * elem_bytes(dtype);
  const size_t vbytes = (size_t)bh * (size_t)n * sizeof(float);
  if (overlap(workspace, need, q, tbytes) || overlap(workspace, need, k, tbytes) ||
      overlap(workspace, need, v, tbytes) || overlap(workspace, need, o, tbytes) ||
      overlap(workspace, need, logf, vbytes) || overlap(workspace, need, lse, vbytes) ||
      overlap(workspace, need, c, vbytes))
    return FOX_ERR_INVALID_ARG;
  return from_hip(fox::launch_attn_fwd_pruned(q, k, v, logf, o, lse, c, static_cast<float*>(workspace), bh, (int)n,
                                              (int)d, scale, dtype == FOX_BF16, stream));
}

size_t fox_attn_decode_workspace_bytes(int64_t s, int64_t h, int64_t l, int64_t d) {
  if (s <= 0 || h <= 0 || l <= 0 || l > FOX_MAX_SEQ || !head_dim_ok(d) || s > kI32Max / h) return 0;
  return fox::decode_workspace_bytes(s * h, (int)l, (int)d);
}

size_t fox_attn_bwd_workspace_bytes(int64_t b, int64_t h, int64_t n, int64_t d) {
  if (b <= 0 || h <= 0 || n <= 0 || n > FOX_MAX_SEQ || !head_dim_ok(d) || b > kI32Max / h) return 0;
  return fox::attn_bwd_workspace_bytes(b * h, (int)n, (int)d);
}

fox_status_t fox_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                          const float* lse, const float* logf, void* dq, void* dk, void* dv, float* dlogf,
                          void* workspace, size_t workspace_bytes, int64_t b, int64_t h, int64_t n, int64_t d,
                          float scale, fox_dtype_t dtype, int causal, hipStream_t stream) {
  return fox_attn_bwd_ex(q, k, v, o, dout, lse, logf, dq, dk, dv, dlogf, workspace, workspace_bytes, b, h, n, d,
                         scale, dtype, causal, FOX_HEAD_MAJOR, stream);
}

// Validation shared by the backward entry points; need: the workspace bytes the call uses.
static fox_status_t bwd_args(const void* q, const void* k, const void* v, const void* o, const void* dout,
                             const float* lse, const float* logf, void* dq, void* dk, void* dv, float* dlogf,
                             void* workspace, size_t workspace_bytes, int64_t b, int64_t h, int64_t n, int64_t d,
                             float scale, fox_dtype_t dtype, fox_layout_t layout, size_t need) {
  if (!q || !k || !v || !o || !dout || !lse || !logf || !dq || !dk || !dv || !dlogf) return FOX_ERR_INVALID_ARG;
  if (b <= 0 || h <= 0 || n <= 0 || d <= 0 || n > FOX_MAX_SEQ) return FOX_ERR_INVALID_ARG;
  if (b > kI32Max / h) return FOX_ERR_INVALID_ARG;
  if (!dtype_ok(dtype) || !head_dim_ok(d)) return FOX_ERR_UNSUPPORTED;
  if (!scale_ok(scale)) return FOX_ERR_INVALID_ARG;
  const int64_t block_rows = dtype == FOX_F32 ? 64 : 128;  // rows per workgroup along the grid's y
  if ((n + block_rows - 1) / block_rows > kMaxGridY) return FOX_ERR_INVALID_ARG;
  if (layout != FOX_HEAD_MAJOR && layout != FOX_TOKEN_MAJOR) return FOX_ERR_UNSUPPORTED;
  // token-major: one head's rows span (n-1)*h*d + d elements, addressed with 32-bit byte offsets
  if (layout == FOX_TOKEN_MAJOR && (n + 256) * h * d * (int64_t)elem_bytes(dtype) > kI32Max)
    return FOX_ERR_UNSUPPORTED;
  const void* t16[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* p : t16)
    if (!aligned(p, 16)) return FOX_ERR_INVALID_ARG;
  if (!aligned(lse, 4) || !aligned(logf, 4) || !aligned(dlogf, 4)) return FOX_ERR_INVALID_ARG;
  const int64_t bh = b * h;
  if (!workspace || !aligned(workspace, 16) || workspace_bytes < need) return FOX_ERR_WORKSPACE;
  const size_t tb = (size_t)bh * (size_t)n * (size_t)d * elem_bytes(dtype), vb = (size_t)bh * (size_t)n * sizeof(float);
  // every output (and the workspace) apart from every other buffer
  const void* outs[] = {dq, dk, dv, dlogf, workspace};
  const size_t osz[] = {tb, tb, tb, vb, need};
  const void* all[] = {q, k, v, o, dout, lse, logf, dq, dk, dv, dlogf, workspace};
  const size_t asz[] = {tb, tb, tb, tb, tb, vb, vb, tb, tb, tb, vb, need};
  for (int i = 0; i < 5; ++i)  // outs[i] is all[7 + i]
    for (int j = 0; j < 12; ++j)
      if (j != 7 + i && overlap(outs[i], osz[i], all[j], asz[j])) return FOX_ERR_INVALID_ARG;
  return FOX_OK;
}

fox_status_t fox_attn_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
                             const float* lse, const float* logf, void* dq, void* dk, void* dv, float* dlogf,
                             void* workspace, size_t workspace_bytes, int64_t b, int64_t h, int64_t n, int64_t d,
                             float scale, fox_dtype_t dtype, int causal, fox_layout_t layout, hipStream_t stream) {
  const size_t need = fox_attn_bwd_workspace_bytes(b, h, n, d);
  const fox_status_t st = bwd_args(q, k, v, o, dout, lse, logf, dq, dk, dv, dlogf, workspace, workspace_bytes, b, h,
                                   n, d, scale, dtype, layout, need);
  if (st != FOX_OK) return st;
  if (dtype == FOX_F32)
    return from_hip(fox::launch_attn_bwd_f32(
        static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
        static_cast<const float*>(o), static_cast<const float*>(dout), lse, logf, static_cast<float*>(dq),
        static_cast<float*>(dk), static_cast<float*>(dv), dlogf, workspace, b, h, (int)n, (int)d, scale, causal != 0,
        layout == FOX_TOKEN_MAJOR, stream));
  return from_hip(fox::launch_attn_bwd(q, k, v, o, dout, lse, logf, dq, dk, dv, dlogf, workspace, b, h, (int)n,
                                       (int)d, scale, causal != 0, layout == FOX_TOKEN_MAJOR, stream));
}

// The staged dS of one head is addressed with 32-bit byte offsets.
static bool staged_size_ok(int64_t n) { return fox::attn_bwd_staged_head_bytes((int)n) <= kI32Max; }

size_t fox_attn_bwd_staged_workspace_bytes(int64_t b, int64_t h, int64_t n, int64_t d) {
  if (b <= 0 || h <= 0 || n <= 0 || n > FOX_MAX_SEQ || d != 128 || b > kI32Max / h || !staged_size_ok(n)) return 0;
  return fox::attn_bwd_staged_workspace_bytes(b * h, (int)n);
}

fox_status_t fox_attn_bwd_staged(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                 const float* lse, const float* logf, void* dq, void* dk, void* dv, float* dlogf,
                                 void* workspace, size_t workspace_bytes, int64_t b, int64_t h, int64_t n, int64_t d,
                                 float scale, fox_dtype_t dtype, fox_layout_t layout, hipStream_t stream) {
  const size_t need = fox_attn_bwd_staged_workspace_bytes(b, h, n, d);
  const fox_status_t st = bwd_args(q, k, v, o, dout, lse, logf, dq, dk, dv, dlogf, workspace, workspace_bytes, b, h,
                                   n, d, scale, dtype, layout, need);
  if (st != FOX_OK) return st;
  if (dtype != FOX_BF16 || d != 128 || !staged_size_ok(n)) return FOX_ERR_UNSUPPORTED;
  return from_hip(fox::launch_attn_bwd_staged(q, k, v, o, dout, lse, logf, dq, dk, dv, dlogf, workspace, b, h, (int)n,
                                              scale, layout == FOX_TOKEN_MAJOR, stream));
}

// Validation shared by the decode entry points (cache_lens: the ragged step's lengths, or null;
// ws_required false: no caller workspace, the split records go to the library's scratch).
static fox_status_t decode_args(const void* q, const void* k_cache, const void* v_cache, float* c_cache,
                                const float* logf_new, const int32_t* cache_lens, void* o, float* lse, void* workspace,
                                size_t workspace_bytes, int64_t s, int64_t h, int64_t l, int64_t d, float scale,
                                fox_dtype_t dtype, bool ws_required = true) {
  if (!q || !k_cache || !v_cache || !c_cache || !logf_new || !o) return FOX_ERR_INVALID_ARG;
  if (s <= 0 || h <= 0 || l <= 0 || d <= 0 || l > FOX_MAX_SEQ) return FOX_ERR_INVALID_ARG;
  if (s > kI32Max / h) return FOX_ERR_INVALID_ARG;
  if (!dtype_ok(dtype) || !head_dim_ok(d)) return FOX_ERR_UNSUPPORTED;
  if (!scale_ok(scale)) return FOX_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16))
    return FOX_ERR_INVALID_ARG;
  if (!aligned(c_cache, 4) || !aligned(logf_new, 4) || !aligned(lse, 4) || !aligned(cache_lens, 4))
    return FOX_ERR_INVALID_ARG;
  const int64_t sh = s * h;
  const int nsplit = fox::decode_num_splits(sh, (int)l, (int)d);
  if (sh > kI32Max / nsplit) return FOX_ERR_INVALID_ARG;
  const size_t need = fox::decode_workspace_bytes(sh, (int)l, (int)d);
  if (ws_required && (!workspace || !aligned(workspace, 16) || workspace_bytes < need)) return FOX_ERR_WORKSPACE;
  const size_t eb = elem_bytes(dtype);
  const size_t obytes = (size_t)sh * (size_t)d * eb, cbytes = (size_t)sh * (size_t)l * sizeof(float);
  const size_t kvbytes = (size_t)sh * (size_t)l * (size_t)d * eb, sbytes = (size_t)sh * sizeof(float);
  const size_t lbytes = (size_t)s * sizeof(int32_t);
  // every buffer written (o, lse, c_cache, workspace) apart from every other buffer
  const void* outs[] = {o, lse, c_cache, workspace};
  const size_t osz[] = {obytes, sbytes, cbytes, need};
  const void* all[] = {q, k_cache, v_cache, c_cache, logf_new, cache_lens, o, lse, workspace};
  const size_t asz[] = {obytes, kvbytes, kvbytes, cbytes, sbytes, lbytes, obytes, sbytes, need};
  const int self[] = {6, 7, 3, 8};  // outs[i] is all[self[i]]
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 9; ++j)
      if (j != self[i] && overlap(outs[i], osz[i], all[j], asz[j])) return FOX_ERR_INVALID_ARG;
  return FOX_OK;
}

fox_status_t fox_attn_decode(const void* q, const void* k_cache, const void* v_cache, float* c_cache,
                             const float* logf_new, void* o, float* lse, void* workspace, size_t workspace_bytes,
                             int64_t s, int64_t h, int64_t l, int64_t d, float scale, fox_dtype_t dtype,
                             hipStream_t stream) {
  const fox_status_t st = decode_args(q, k_cache, v_cache, c_cache, logf_new, nullptr, o, lse, workspace,
                                      workspace_bytes, s, h, l, d, scale, dtype);
  if (st != FOX_OK) return st;
  return from_hip(fox::launch_attn_decode(q, k_cache, v_cache, c_cache, logf_new, nullptr, (int)h, o, lse,
                                          static_cast<float*>(workspace), s * h, (int)l, (int)d, scale,
                                          dtype == FOX_BF16, stream));
}

fox_status_t fox_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, float* c_cache,
                                     const float* logf_new, void* o, float* lse, int64_t s, int64_t h, int64_t l,
                                     int64_t d, float scale, fox_dtype_t dtype, hipStream_t stream) {
  const fox_status_t st = decode_args(q, k_cache, v_cache, c_cache, logf_new, nullptr, o, lse, nullptr, 0, s, h, l, d,
                                      scale, dtype, false);
  if (st != FOX_OK) return st;
  if (fox::decode_workspace_bytes(s * h, (int)l, (int)d) > (size_t)FOX_DECODE_SCRATCH_BYTES) return FOX_ERR_SCRATCH;
  float* ws = nullptr;
  const hipError_t e = fox::decode_scratch(&ws);
  if (e != hipSuccess) return FOX_ERR_HIP;
  return from_hip(fox::launch_attn_decode(q, k_cache, v_cache, c_cache, logf_new, nullptr, (int)h, o, lse, ws, s * h,
                                          (int)l, (int)d, scale, dtype == FOX_BF16, stream));
}

fox_status_t fox_attn_decode_ragged(const void* q, const void* k_cache, const void* v_cache, float* c_cache,
                                    const float* logf_new, const int32_t* cache_lens, void* o, float* lse,
                                    void* workspace, size_t workspace_bytes, int64_t s, int64_t h, int64_t l,
                                    int64_t d, float scale, fox_dtype_t dtype, hipStream_t stream) {
  if (!cache_lens) return FOX_ERR_INVALID_ARG;
  const fox_status_t st = decode_args(q, k_cache, v_cache, c_cache, logf_new, cache_lens, o, lse, workspace,
                                      workspace_bytes, s, h, l, d, scale, dtype);
  if (st != FOX_OK) return st;
  return from_hip(fox::launch_attn_decode(q, k_cache, v_cache, c_cache, logf_new, cache_lens, (int)h, o, lse,
                                          static_cast<float*>(workspace), s * h, (int)l, (int)d, scale,
                                          dtype == FOX_BF16, stream));
}

fox_status_t fox_attn_decode_paged(const void* q, const void* k_pages, const void* v_pages, float* c_pages,
                                   const int32_t* block_table, const int32_t* cache_lens, const float* logf_new,
                                   void* o, float* lse, void* workspace, size_t workspace_bytes, int64_t s,
                                   int64_t h, int64_t num_pages, int64_t page_size, int64_t max_pages, int64_t d,
                                   float scale, fox_dtype_t dtype, hipStream_t stream) {
  if (!q || !k_pages || !v_pages || !c_pages || !block_table || !cache_lens || !logf_new || !o)
    return FOX_ERR_INVALID_ARG;
  if (s <= 0 || h <= 0 || num_pages <= 0 || max_pages <= 0 || d <= 0) return FOX_ERR_INVALID_ARG;
  if (page_size < 16 || page_size > 4096 || (page_size & (page_size - 1)) != 0) return FOX_ERR_INVALID_ARG;
  if (max_pages > FOX_MAX_SEQ / page_size || num_pages > kI32Max || s > kI32Max / h) return FOX_ERR_INVALID_ARG;
  if (!dtype_ok(dtype) || !head_dim_ok(d)) return FOX_ERR_UNSUPPORTED;
  if (!scale_ok(scale)) return FOX_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) || !aligned(o, 16)) return FOX_ERR_INVALID_ARG;
  if (!aligned(c_pages, 4) || !aligned(block_table, 4) || !aligned(cache_lens, 4) || !aligned(logf_new, 4) ||
      !aligned(lse, 4))
    return FOX_ERR_INVALID_ARG;
  const int64_t sh = s * h, l = max_pages * page_size;
  const int nsplit = fox::decode_num_splits(sh, (int)l, (int)d);
  if (sh > kI32Max / nsplit) return FOX_ERR_INVALID_ARG;
  const size_t need = fox::decode_workspace_bytes(sh, (int)l, (int)d);
  if (!workspace || !aligned(workspace, 16) || workspace_bytes < need) return FOX_ERR_WORKSPACE;
  const size_t eb = elem_bytes(dtype), slots = (size_t)num_pages * (size_t)h * (size_t)page_size;
  const size_t obytes = (size_t)sh * (size_t)d * eb, sbytes = (size_t)sh * sizeof(float);
  const size_t kvbytes = slots * (size_t)d * eb, cbytes = slots * sizeof(float);
  const size_t tbytes = (size_t)s * (size_t)max_pages * sizeof(int32_t), lbytes = (size_t)s * sizeof(int32_t);
  // every buffer written (o, lse, c_pages, workspace) apart from every other buffer
  const void* outs[] = {o, lse, c_pages, workspace};
  const size_t osz[] = {obytes, sbytes, cbytes, need};
  const void* all[] = {q, k_pages, v_pages, c_pages, block_table, cache_lens, logf_new, o, lse, workspace};
  const size_t asz[] = {obytes, kvbytes, kvbytes, cbytes, tbytes, lbytes, sbytes, obytes, sbytes, need};
  const int self[] = {7, 8, 3, 9};  // outs[i] is all[self[i]]
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 10; ++j)
      if (j != self[i] && overlap(outs[i], osz[i], all[j], asz[j])) return FOX_ERR_INVALID_ARG;
  int shift = 0;
  while ((int64_t{1} << shift) < page_size) ++shift;
  return from_hip(fox::launch_attn_decode_paged(q, k_pages, v_pages, c_pages, block_table, (int)max_pages, shift,
                                                (int)num_pages, logf_new, cache_lens, (int)h, o, lse,
                                                static_cast<float*>(workspace), sh, (int)d, scale, dtype == FOX_BF16,
                                                stream));
}

}  // extern "C"
