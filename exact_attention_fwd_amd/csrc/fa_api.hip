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

// Two fp32 per query row: D_i, then LSE_i · log2(e), each array rounded up to 256 bytes.
size_t backward_workspace_bytes(long long rows) {
  if (rows < 0) return 0;
  return 2 * round256((size_t)rows * sizeof(float));
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
    case FA_ERR_SCRATCH_TOO_SMALL:
      return "FA_ERR_SCRATCH_TOO_SMALL: the problem needs more than the library's 16 MiB static scratch";
  }
  return "unknown fa_status";
}

const char* fa_last_hip_error(void) { return g_last_hip_error; }

int fa_version(void) { return 10000; }

// Checks shared by the dense and packed forms.  `rows_max` is the longest
// sequence, `stride_rows` the row count a buffer descriptor of one head spans
// (N for dense, max_seqlen for packed), `row_elems` the elements per row of
// the widest tensor (d dense, H*d packed).
static fa_status check_common(int B, int H, int Hkv, int d, long long rows_max, long long row_elems, float scale) {
  if (B <= 0 || H <= 0 || Hkv <= 0 || d <= 0 || rows_max < 0) return FA_ERR_BAD_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (H % Hkv != 0) return FA_ERR_BAD_SHAPE;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_BAD_SHAPE;
  if ((long long)B * H > INT_MAX / 4) return FA_ERR_BAD_SHAPE;
  if ((rows_max + 127) / 128 * (long long)B * H > INT_MAX / 2) return FA_ERR_BAD_SHAPE;
  if (rows_max * row_elems * 2 >= (1LL << 31)) return FA_ERR_BAD_SHAPE;  // 32-bit buffer offsets per head
  return FA_OK;
}

static fa_status forward_impl(fa_dtype dt, fa::AttnShape sh, int d, const void* q, const void* k, const void* v,
                              void* o, float* lse, int causal, float scale, void* stream,
                              fa::RopeArgs rope = fa::RopeArgs{}) {
  if (dt != FA_F32 && dt != FA_BF16) return FA_ERR_UNSUPPORTED;
  const bool packed = sh.cu != nullptr;
  fa_status st = check_common(sh.B, sh.H, sh.Hkv, d, sh.N, packed ? (long long)sh.H * d : d, scale);
  if (st != FA_OK) return st;
  if (packed && sh.total < 0) return FA_ERR_BAD_SHAPE;
  if (!packed && !fits(sh.B, sh.H, sh.N, d)) return FA_ERR_BAD_SHAPE;
  if (dt == FA_F32 && (long long)sh.B * sh.H > 65535) return FA_ERR_BAD_SHAPE;  // grid.y limit of the fp32 path
  if (sh.N == 0 || (packed && sh.total == 0)) return FA_OK;
  if (!q || !k || !v || !o) return FA_ERR_NULL_PTR;
  st = device_ready();
  if (st != FA_OK) return st;
  fa::ForwardArgs a{dt == FA_BF16, sh, fa::PagedKV{}, rope, d, q, k, v, o, lse, causal != 0, scale,
                    (hipStream_t)stream};
  return hip_status(fa::launch_forward(a));
}

fa_status fa_forward(fa_dtype dt, int B, int H, int N, int d, const void* q, const void* k, const void* v, void* o,
                     float* lse, int causal, float scale, void* stream) {
  return forward_impl(dt, fa::AttnShape{B, H, H, N, 0, nullptr}, d, q, k, v, o, lse, causal, scale, stream);
}

fa_status fa_forward_gqa(fa_dtype dt, int B, int H, int Hkv, int N, int d, const void* q, const void* k,
                         const void* v, void* o, float* lse, int causal, float scale, void* stream) {
  return forward_impl(dt, fa::AttnShape{B, H, Hkv, N, 0, nullptr}, d, q, k, v, o, lse, causal, scale, stream);
}

fa_status fa_forward_varlen(fa_dtype dt, int B, int H, int Hkv, int max_seqlen, int total, int d,
                            const int32_t* cu_seqlens, const void* q, const void* k, const void* v, void* o,
                            float* lse, int causal, float scale, void* stream) {
  if (!cu_seqlens && B > 0) return FA_ERR_NULL_PTR;
  return forward_impl(dt, fa::AttnShape{B, H, Hkv, max_seqlen, total, cu_seqlens}, d, q, k, v, o, lse, causal,
                      scale, stream);
}

// Rotary tables: both or neither, 16-byte aligned, at least one row.
static fa_status check_rope(const float* cos_t, const float* sin_t, int rows, fa::RopeArgs& out) {
  out = fa::RopeArgs{};
  if (!cos_t && !sin_t) return FA_OK;
  if (!cos_t || !sin_t) return FA_ERR_NULL_PTR;
  if (rows <= 0 || (reinterpret_cast<uintptr_t>(cos_t) & 15) || (reinterpret_cast<uintptr_t>(sin_t) & 15))
    return FA_ERR_BAD_SHAPE;
  out = fa::RopeArgs{cos_t, sin_t, rows, 0};
  return FA_OK;
}

fa_status fa_forward_rope(fa_dtype dt, int B, int H, int Hkv, int N, int total, int d, const int32_t* cu_seqlens,
                          const void* q, const void* k, const void* v, void* o, float* lse, int causal, float scale,
                          const float* rope_cos, const float* rope_sin, int rope_rows, int rope_interleaved,
                          void* stream) {
  if (dt != FA_BF16) return FA_ERR_UNSUPPORTED;
  fa::RopeArgs rope;
  fa_status st = check_rope(rope_cos, rope_sin, rope_rows, rope);
  if (st != FA_OK) return st;
  if (!rope.cos) return FA_ERR_NULL_PTR;
  if (rope_rows < N) return FA_ERR_BAD_SHAPE;  // every position 0 .. N-1 needs a row
  rope.interleaved = rope_interleaved != 0;
  return forward_impl(dt, fa::AttnShape{B, H, Hkv, N, cu_seqlens ? total : 0, cu_seqlens}, d, q, k, v, o, lse,
                      causal, scale, stream, rope);
}

fa_status fa_prefill_paged(int B, int H, int Hkv, int d, int max_seqlen_q, int total_q,
                           const int32_t* cu_seqlens_q, const void* q, const void* kv_pool, int page_size,
                           int num_pages, const int32_t* block_table, int max_blocks_per_seq,
                           const int32_t* seq_lens_k, void* o, float* lse, int causal, float scale,
                           const float* rope_cos, const float* rope_sin, int rope_rows, int rope_interleaved,
                           void* stream) {
  fa_status st = check_common(B, H, Hkv, d, max_seqlen_q, (long long)H * d, scale);
  if (st != FA_OK) return st;
  fa::RopeArgs rope;
  st = check_rope(rope_cos, rope_sin, rope_rows, rope);
  if (st != FA_OK) return st;
  rope.interleaved = rope_interleaved != 0;
  if (total_q < 0 || num_pages <= 0 || max_blocks_per_seq <= 0) return FA_ERR_BAD_SHAPE;
  if (page_size != 256) return FA_ERR_UNSUPPORTED;
  if (max_blocks_per_seq > fa::kMaxPrefillPages) return FA_ERR_UNSUPPORTED;
  if (!fits(num_pages, 2, page_size, (long long)Hkv * d)) return FA_ERR_BAD_SHAPE;
  if (max_seqlen_q == 0 || total_q == 0) return FA_OK;
  if (!cu_seqlens_q || !q || !kv_pool || !block_table || !seq_lens_k || !o) return FA_ERR_NULL_PTR;
  st = device_ready();
  if (st != FA_OK) return st;
  fa::ForwardArgs a{true,
                    fa::AttnShape{B, H, Hkv, max_seqlen_q, total_q, cu_seqlens_q},
                    fa::PagedKV{kv_pool, block_table, seq_lens_k, max_blocks_per_seq, num_pages},
                    rope, d, q, nullptr, nullptr, o, lse, causal != 0, scale, (hipStream_t)stream};
  return hip_status(fa::launch_forward(a));
}

size_t fa_backward_workspace_bytes(int B, int H, int N, int d) {
  (void)d;
  if (B <= 0 || H <= 0 || N < 0) return 0;
  return fa::backward_workspace_bytes((long long)B * H * N);
}

size_t fa_backward_varlen_workspace_bytes(int H, int total, int d) {
  (void)d;
  if (H <= 0 || total < 0) return 0;
  return fa::backward_workspace_bytes((long long)H * total);
}

static fa_status backward_impl(fa_dtype dt, fa::AttnShape sh, int d, const void* q, const void* k, const void* v,
                               const void* o, const void* dout, const float* lse, void* dq, void* dk, void* dv,
                               void* workspace, size_t workspace_bytes, int causal, float scale, void* stream) {
  if (dt != FA_BF16) return FA_ERR_UNSUPPORTED;
  const bool packed = sh.cu != nullptr;
  fa_status st = check_common(sh.B, sh.H, sh.Hkv, d, sh.N, packed ? (long long)sh.H * d : d, scale);
  if (st != FA_OK) return st;
  if (packed && sh.total < 0) return FA_ERR_BAD_SHAPE;
  if (!packed && !fits(sh.B, sh.H, sh.N, d)) return FA_ERR_BAD_SHAPE;
  if (sh.N == 0 || (packed && sh.total == 0)) return FA_OK;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL_PTR;
  const long long rows = packed ? (long long)sh.H * sh.total : (long long)sh.B * sh.H * sh.N;
  if (!workspace || workspace_bytes < fa::backward_workspace_bytes(rows)) return FA_ERR_WORKSPACE;
  st = device_ready();
  if (st != FA_OK) return st;
  float* const ws = static_cast<float*>(workspace);
  fa::BackwardArgs a{sh, d, q, k, v, o, dout, lse, dq, dk, dv, ws, ws + round256((size_t)rows * sizeof(float)) / sizeof(float),
                     causal != 0, scale,
                     (hipStream_t)stream};
  return hip_status(fa::launch_backward(a));
}

fa_status fa_backward(fa_dtype dt, int B, int H, int N, int d, const void* q, const void* k, const void* v,
                      const void* o, const void* dout, const float* lse, void* dq, void* dk, void* dv,
                      void* workspace, size_t workspace_bytes, int causal, float scale, void* stream) {
  return backward_impl(dt, fa::AttnShape{B, H, H, N, 0, nullptr}, d, q, k, v, o, dout, lse, dq, dk, dv, workspace,
                       workspace_bytes, causal, scale, stream);
}

fa_status fa_backward_gqa(fa_dtype dt, int B, int H, int Hkv, int N, int d, const void* q, const void* k,
                          const void* v, const void* o, const void* dout, const float* lse, void* dq, void* dk,
                          void* dv, void* workspace, size_t workspace_bytes, int causal, float scale, void* stream) {
  return backward_impl(dt, fa::AttnShape{B, H, Hkv, N, 0, nullptr}, d, q, k, v, o, dout, lse, dq, dk, dv, workspace,
                       workspace_bytes, causal, scale, stream);
}

fa_status fa_backward_varlen(fa_dtype dt, int B, int H, int Hkv, int max_seqlen, int total, int d,
                             const int32_t* cu_seqlens, const void* q, const void* k, const void* v, const void* o,
                             const void* dout, const float* lse, void* dq, void* dk, void* dv, void* workspace,
                             size_t workspace_bytes, int causal, float scale, void* stream) {
  if (!cu_seqlens && B > 0) return FA_ERR_NULL_PTR;
  return backward_impl(dt, fa::AttnShape{B, H, Hkv, max_seqlen, total, cu_seqlens}, d, q, k, v, o, dout, lse, dq, dk,
                       dv, workspace, workspace_bytes, causal, scale, stream);
}

size_t fa_decode_workspace_bytes(int num_seqs, int H, int d, int max_blocks_per_seq) {
  return fa::decode_workspace_bytes(num_seqs, H, d, max_blocks_per_seq);
}

// Checks shared by the decode entry points (everything but the workspace).
static fa_status decode_check(int num_seqs, int H, int Hkv, int d, int page_size, int num_pages,
                              int max_blocks_per_seq, const void* q, const void* kv_pool,
                              const int32_t* block_table, const int32_t* seq_lens, void* o, float scale) {
  if (num_seqs <= 0 || H <= 0 || Hkv <= 0 || d <= 0 || page_size <= 0 || num_pages <= 0 || max_blocks_per_seq <= 0)
    return FA_ERR_BAD_SHAPE;
  if (H % Hkv != 0) return FA_ERR_BAD_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (page_size != 256) return FA_ERR_UNSUPPORTED;
  const long long hblocks = (H / Hkv + 31) / 32;  // query-head blocks per key/value head (grouped kernel)
  if (H > 4096 || !fits(num_pages, 2, page_size, (long long)Hkv * d) ||
      !fits(num_seqs, H, max_blocks_per_seq, d + 2) || (long long)max_blocks_per_seq * page_size > INT_MAX ||
      (long long)num_seqs * max_blocks_per_seq * 2 * H > INT_MAX ||  // grid of the split kernel
      (long long)num_seqs * max_blocks_per_seq * 2 * Hkv * hblocks > INT_MAX)  // waves of the grouped kernel
    return FA_ERR_BAD_SHAPE;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_BAD_SHAPE;
  if (!q || !kv_pool || !block_table || !seq_lens || !o) return FA_ERR_NULL_PTR;
  return FA_OK;
}

static fa_status decode_impl(int num_seqs, int H, int Hkv, int d, int page_size, int num_pages,
                             int max_blocks_per_seq, const void* q, const void* kv_pool, const int32_t* block_table,
                             const int32_t* seq_lens, void* o, float* lse, float scale, void* workspace,
                             size_t workspace_bytes, void* stream) {
  fa_status st = decode_check(num_seqs, H, Hkv, d, page_size, num_pages, max_blocks_per_seq, q, kv_pool,
                              block_table, seq_lens, o, scale);
  if (st != FA_OK) return st;
  if (!workspace || workspace_bytes < fa::decode_workspace_bytes(num_seqs, H, d, max_blocks_per_seq))
    return FA_ERR_WORKSPACE;
  st = device_ready();
  if (st != FA_OK) return st;
  fa::DecodeArgs a{num_seqs, H, Hkv, d, page_size, num_pages, max_blocks_per_seq, q, kv_pool, block_table, seq_lens,
                   o, lse, scale, static_cast<float*>(workspace), (hipStream_t)stream};
  return hip_status(fa::launch_decode(a));
}

fa_status fa_decode_paged(int num_seqs, int H, int d, int page_size, int num_pages, int max_blocks_per_seq,
                          const void* q, const void* kv_pool, const int32_t* block_table, const int32_t* seq_lens,
                          void* o, float* lse, float scale, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(num_seqs, H, H, d, page_size, num_pages, max_blocks_per_seq, q, kv_pool, block_table, seq_lens,
                     o, lse, scale, workspace, workspace_bytes, stream);
}

fa_status fa_decode_paged_gqa(int num_seqs, int H, int Hkv, int d, int page_size, int num_pages,
                              int max_blocks_per_seq, const void* q, const void* kv_pool,
                              const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse, float scale,
                              void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(num_seqs, H, Hkv, d, page_size, num_pages, max_blocks_per_seq, q, kv_pool, block_table,
                     seq_lens, o, lse, scale, workspace, workspace_bytes, stream);
}

size_t fa_decode_static_scratch_bytes(void) { return fa::kStaticScratchBytes; }

fa_status fa_decode_paged_gqa_static(int num_seqs, int H, int Hkv, int d, int page_size, int num_pages,
                                     int max_blocks_per_seq, const void* q, const void* kv_pool,
                                     const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse,
                                     float scale, void* stream) {
  fa_status st = decode_check(num_seqs, H, Hkv, d, page_size, num_pages, max_blocks_per_seq, q, kv_pool,
                              block_table, seq_lens, o, scale);
  if (st != FA_OK) return st;
  if (fa::decode_workspace_bytes(num_seqs, H, d, max_blocks_per_seq) > fa::kStaticScratchBytes)
    return FA_ERR_SCRATCH_TOO_SMALL;
  st = device_ready();
  if (st != FA_OK) return st;
  void* scratch = nullptr;
  st = hip_status(fa::static_scratch(&scratch));
  if (st != FA_OK) return st;
  fa::DecodeArgs a{num_seqs, H, Hkv, d, page_size, num_pages, max_blocks_per_seq, q, kv_pool, block_table, seq_lens,
                   o, lse, scale, static_cast<float*>(scratch), (hipStream_t)stream};
  return hip_status(fa::launch_decode(a));
}

}  // extern "C"
