// Internal launch interface between the C ABI (fa_api.hip) and the kernel
// translation units.  Arguments reaching these functions are validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Shape of an attention problem as the kernels address it.
//   dense : Q/O [B, H, N, d], K/V [B, Hkv, N, d], LSE/D [B, H, N]
//   varlen: Q/O [total, H, d], K/V [total, Hkv, d], LSE/D [H, total], sequence
//           b owning rows cu[b] .. cu[b+1]-1 (cu on the device), N = max length
// Query head h reads key/value head h / (H / Hkv).
struct AttnShape {
  int B, H, Hkv, N, total;
  const int32_t* cu;  // nullptr: dense
};

// Keys/values read through a page table instead of the query layout: the
// pool is [num_pages, 2 (K, V), 256, Hkv, d]; sequence b owns seq_lens[b]
// keys whose logical page p sits at pool page block_table[b·max_blocks + p].
// Its queries are the last rows of those keys (causal: query i of a sequence
// with n queries sees keys 0 .. i + seq_lens[b] − n).
struct PagedKV {
  const void* pool;  // nullptr: K/V laid out like the queries
  const int32_t* block_table;
  const int32_t* seq_lens;
  int max_blocks, num_pages;
};
constexpr int kMaxPrefillPages = 512;  // block-table entries a paged prefill sequence may use

// Rotary position embedding applied inside the forward: the feature pair
// (x, y) of a row at position p becomes (x·c − y·s, x·s + y·c) with
// c = cos[p][i], s = sin[p][i] (fp32 tables [rows, d/2]).  Pair i is
// (i, i + d/2) (half split) or (2i, 2i+1) (interleaved).  Positions are the
// row's index in its sequence (queries of a paged prefill: i + L − n).
struct RopeArgs {
  const float* cos;  // nullptr: no rotation
  const float* sin;
  int rows;
  int interleaved;
};

struct ForwardArgs {
  bool bf16;
  AttnShape s;
  PagedKV kv;
  RopeArgs rope;
  int d;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int causal;
  float scale;
  hipStream_t stream;
};

struct BackwardArgs {
  AttnShape s;
  int d;
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;  // −D_i, laid out like LSE (workspace)
  float* lse2;   // LSE_i · log2(e), laid out like LSE (workspace)
  int causal;
  float scale;
  hipStream_t stream;
};

struct DecodeArgs {
  int S, H, Hkv, d, page_size, num_pages, max_blocks;
  const void* q;
  const void* kv_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* o;
  float* lse;
  float scale;
  float* part;  // [S, H, splits, d + 2] fp32 workspace (two splits per page, one when Hkv < H)
  hipStream_t stream;
};

hipError_t launch_forward(const ForwardArgs& a);
hipError_t launch_backward(const BackwardArgs& a);
hipError_t launch_decode(const DecodeArgs& a);

// Bytes of the per-device static scratch behind fa_decode_paged_gqa_static.
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
// Device address of this device's static scratch (looked up once per device).
hipError_t static_scratch(void** ptr);

// Workspace sizes (bytes, rounded up to 256).
size_t backward_workspace_bytes(long long rows);  // rows of LSE: B*H*N dense, H*total varlen
size_t decode_workspace_bytes(long long S, long long H, long long d, long long max_blocks);

}  // namespace fa
