// C ABI of the attention library: host-side validation, then launches on the
// caller's stream.  Nothing here allocates device memory or synchronises.
#include <cmath>
#include <climits>

#include "../../include/fa.h"
#include "fa_internal.h"

namespace {

thread_local const char* g_last_hip_error = "no error";

fa_status hip_status(hipError_t e) {
  if (e == hipSuccess) return FA_OK;
  g_last_hip_error = hipGetErrorString(e);
  return FA_ERR_HIP;
}

// A usable device must be current; checked after argument validation so that
// bad arguments are reported the same way with or without a GPU.
fa_status device_ready() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  int count = 0;
  e = hipGetDeviceCount(&count);
  if (e != hipSuccess) return hip_status(e);
  if (count <= 0 || dev < 0) {
    g_last_hip_error = "no HIP device";
    return FA_ERR_HIP;
  }
  return FA_OK;
}

bool fits(long long a, long long b, long long c, long long d) {
  // product of non-negative factors stays below 2^62 elements
  long double p = (long double)a * b * c * d;
  return p < 4.0e18L;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

namespace fa {

size_t backward_workspace_bytes(long long BH, long long N) {
  if (BH <= 0 || N < 0) return 0;
  return round256((size_t)BH * (size_t)N * sizeof(float));
}

size_t decode_workspace_bytes(long long S, long long H, long long d, long long max_blocks) {
  if (S <= 0 || H <= 0 || d <= 0 || max_blocks <= 0) return 0;
  // two 128-token splits per 256-token page
  return round256((size_t)S * H * max_blocks * 2 * (size_t)(d + 2) * sizeof(float));
}

}  // namespace fa

extern "C" {

const char* fa_status_str(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL_PTR: return "FA_ERR_NULL_PTR: a required pointer is NULL";
    case FA_ERR_BAD_SHAPE: return "FA_ERR_BAD_SHAPE: invalid or overflowing size";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head dim, dtype or page size not supported";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
    case FA_ERR_HIP: return "FA_ERR_HIP: HIP runtime error";
  }
  return "unknown fa_status";
}

const char* fa_last_hip_error(void) { return g_last_hip_error; }

int fa_version(void) { return 10000; }

fa_status fa_forward(fa_dtype dt, int B, int H, int N, int d, const void* q, const void* k, const void* v, void* o,
                     float* lse, int causal, float scale, void* stream) {
  if (dt != FA_F32 && dt != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (B <= 0 || H <= 0 || N < 0 || d <= 0) return FA_ERR_BAD_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (!fits(B, H, N, d) || (long long)B * H > INT_MAX / 4 ||
      (long long)((N + 127) / 128) * B * H > INT_MAX / 2)
    return FA_ERR_BAD_SHAPE;
  if (!std::isfinite(scale)) return FA_ERR_BAD_SHAPE;
  if (dt == FA_F32 && (long long)B * H > 65535) return FA_ERR_BAD_SHAPE;  // grid.y limit of the fp32 path
  if (N == 0) return FA_OK;
  if (!q || !k || !v || !o) return FA_ERR_NULL_PTR;
  fa_status st = device_ready();
  if (st != FA_OK) return st;
  fa::ForwardArgs a{dt == FA_BF16, B * H, N, d, q, k, v, o, lse, causal != 0, scale, (hipStream_t)stream};
  return hip_status(fa::launch_forward(a));
}

size_t fa_backward_workspace_bytes(int B, int H, int N, int d) {
  (void)d;
  if (B <= 0 || H <= 0) return 0;
  return fa::backward_workspace_bytes((long long)B * H, N);
}

fa_status fa_backward(fa_dtype dt, int B, int H, int N, int d, const void* q, const void* k, const void* v,
                      const void* o, const void* dout, const float* lse, void* dq, void* dk, void* dv,
                      void* workspace, size_t workspace_bytes, int causal, float scale, void* stream) {
  if (dt != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (B <= 0 || H <= 0 || N < 0 || d <= 0) return FA_ERR_BAD_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (!fits(B, H, N, d) || (long long)B * H > INT_MAX / 4 ||
      (long long)((N + 63) / 64) * B * H > INT_MAX / 2)
    return FA_ERR_BAD_SHAPE;
  if (!std::isfinite(scale)) return FA_ERR_BAD_SHAPE;
  if (N == 0) return FA_OK;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL_PTR;
  if (!workspace || workspace_bytes < fa::backward_workspace_bytes((long long)B * H, N)) return FA_ERR_WORKSPACE;
  fa_status st = device_ready();
  if (st != FA_OK) return st;
  fa::BackwardArgs a{B * H, N, d, q, k, v, o, dout, lse, dq, dk, dv, static_cast<float*>(workspace),
                     causal != 0, scale, (hipStream_t)stream};
  return hip_status(fa::launch_backward(a));
}

size_t fa_decode_workspace_bytes(int num_seqs, int H, int d, int max_blocks_per_seq) {
  return fa::decode_workspace_bytes(num_seqs, H, d, max_blocks_per_seq);
}

fa_status fa_decode_paged(int num_seqs, int H, int d, int page_size, int num_pages, int max_blocks_per_seq,
                          const void* q, const void* kv_pool, const int32_t* block_table, const int32_t* seq_lens,
                          void* o, float* lse, float scale, void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs <= 0 || H <= 0 || d <= 0 || page_size <= 0 || num_pages <= 0 || max_blocks_per_seq <= 0)
    return FA_ERR_BAD_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (page_size != 256) return FA_ERR_UNSUPPORTED;
  if (H > 4096 || !fits(num_pages, 2, page_size, (long long)H * d) ||
      !fits(num_seqs, H, max_blocks_per_seq, d + 2) || (long long)max_blocks_per_seq * page_size > INT_MAX ||
      (long long)num_seqs * max_blocks_per_seq * 2 * H > INT_MAX)  // grid of the split kernel
    return FA_ERR_BAD_SHAPE;
  if (!std::isfinite(scale)) return FA_ERR_BAD_SHAPE;
  if (!q || !kv_pool || !block_table || !seq_lens || !o) return FA_ERR_NULL_PTR;
  if (!workspace || workspace_bytes < fa::decode_workspace_bytes(num_seqs, H, d, max_blocks_per_seq))
    return FA_ERR_WORKSPACE;
  fa_status st = device_ready();
  if (st != FA_OK) return st;
  fa::DecodeArgs a{num_seqs, H, d, page_size, max_blocks_per_seq, q, kv_pool, block_table, seq_lens, o, lse,
                   scale, static_cast<float*>(workspace), (hipStream_t)stream};
  return hip_status(fa::launch_decode(a));
}

}  // extern "C"
