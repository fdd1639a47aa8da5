// Device-side building blocks shared by the gfx950 attention kernels.
//
// Matrix products run on the CDNA4 bf16 MFMA v_mfma_f32_32x32x16_bf16
// (fp32 accumulate).  Its register layout on a 64-lane wavefront, with
// g = lane / 32 and n = lane % 32:
//   A (32 x 16):  lane holds A[n][8g .. 8g+7]        (8 bf16, one 16-byte row piece)
//   B (16 x 32):  lane holds B[8g .. 8g+7][n]
//   C (32 x 32):  lane holds C[8(r/4) + 4g + r%4][n]  for r = 0..15
// so a C tile is "one column per lane, 16 of its 32 rows per lane".
//
// Chaining two products (C of the first becomes the B operand of the second,
// contracting over C's rows) needs C's row order to match B's k order.  The
// first product therefore reads its A rows through perm_row(), which swaps
// bits 2 and 3 of the row index: then register r of C in lane (g, n) holds
// row 16(r/8) + 8g + r%8, and registers 8h..8h+7 of a lane are exactly the
// B-operand k-slots 8g..8g+7 of the k-step covering rows 16h..16h+15.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();
constexpr float kNaN = __builtin_nanf("");

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
// log2(x) on the transcendental unit (v_log_f32).
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Row permutation inside a 32-row MFMA block: swap bits 2 and 3 (an involution).
__device__ __forceinline__ int perm_row(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// Combine a per-lane value with the one held by lane ^ 32 (v_permlane32_swap):
// swapping x with itself leaves (x[l], x[l^32]) in the two results of lane l.
__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Round two fp32 to bf16 (nearest-even, v_cvt_pk_bf16_f32) and pack them.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (bf16)lo;
  v[1] = (bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 pack8(const float* p) {
  u32x4 w;
  w[0] = pack_bf16x2(p[0], p[1]);
  w[1] = pack_bf16x2(p[2], p[3]);
  w[2] = pack_bf16x2(p[4], p[5]);
  w[3] = pack_bf16x2(p[6], p[7]);
  return __builtin_bit_cast(bf16x8, w);
}

// K/V (and Q/dO in the backward) are staged through LDS in tiles of 64 rows.
constexpr int kTileRows = 64;

// XOR swizzle of the 16-byte chunks of a row-major [64][D] tile read as a
// row-major MFMA operand: 16 lanes take rows perm_row(m), one chunk each, and
// rm_swz() maps those rows to 16 (D=128) / 8 (D=64) distinct chunks.
template <int D>
__device__ __forceinline__ int rm_swz(int r) {
  return D >= 128 ? (perm_row(r) & 15) : (perm_row(r) & 7);
}

// Swizzle of the row-major V tile (16-byte chunk c of row r lives at
// c ^ v_swz(r)).  A transposed operand read covers four consecutive rows per
// 16-lane group and 16 columns per group pair; the pattern {0, 10, 4, 14} on
// r % 4 sends those pieces to distinct banks whether the LDS serves 16 or 32
// lanes of an 8-byte read per cycle.
template <int D>
__device__ __forceinline__ int v_swz(int row) {
  return ((0xE4A0 >> (4 * (row & 3))) & 15) & (D / 8 - 1);
}

// ---------------------------------------------------------------------------
// Buffer resources: 128-bit descriptors over one contiguous byte range.  Raw
// buffer loads past `bytes` return zeros in hardware, so tile loads need no
// bounds branches.  (Word 3 = 0x00020000 is the CDNA data-format word for raw
// 32-bit access.)
// ---------------------------------------------------------------------------
// Every descriptor in this library covers a range that is the same for the
// whole wavefront; reading base and size through readfirstlane states that,
// so the descriptor is built in scalar registers (a free move when they
// already are) and loads through it never need a per-lane waterfall loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
// Same load with the non-temporal hint: data read once (streamed through).
__device__ __forceinline__ u32x4 buf_load16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2));
}

typedef __attribute__((address_space(3))) void lds_void;
// Direct HBM -> LDS load of 16 bytes per lane: lane l's bytes land at
// lds_wave_base + 16*l (the destination is one contiguous 1 KiB block per
// wavefront instruction); `off` is this lane's byte offset in the buffer.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, void* lds_wave_base, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_wave_base, 16, (int)off, 0, 0, 0);
}
// Wait until every direct-to-LDS load this wavefront issued has landed.
__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// (i & 3) of the 4-element pieces addressed by lanes 4t + (i >> 2), t = 0..3.
// If lane j of the group addresses row (r0 + j/4), columns c0 + 4(j%4) ..+3 of
// a row-major tile, lane i receives rows r0..r0+3 of column c0 + i.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
__device__ __forceinline__ bf16x4 lds_read_tr4(const bf16* p) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p)));
}

// Swizzle for a row-major [64][D] tile that is read both as a row-major MFMA
// operand (rows perm_row(m) of 16 lanes, one 16-byte chunk each) and through
// transposed reads (4 consecutive rows x 4 consecutive chunks per 32 lanes):
// chunk c of row r lives at c ^ dual_swz(r).  The XOR-linear map below keeps
// both patterns free of bank conflicts for 16- and 32-lane LDS service.
template <int D>
__device__ __forceinline__ int dual_swz(int r) {
  constexpr int b0 = D >= 128 ? 4 : 2, b1 = D >= 128 ? 10 : 4, b2 = 1, b3 = 3;
  return ((r & 1) ? b0 : 0) ^ ((r & 2) ? b1 : 0) ^ ((r & 4) ? b2 : 0) ^ ((r & 8) ? b3 : 0);
}

// Addressing of one (batch, query head) unit: element offsets of row 0 in
// Q/O (and dQ/dO), in K/V (and dK/dV) and in LSE/D, the row strides in
// elements, and the sequence length.  `cut` is set when a packed sequence is
// longer than the launch's maximum length: its rows past that length are not
// computed, so the rows that are get NaN outputs (the call's error made
// visible instead of a silently partial result).
struct HeadView {
  size_t q_off, kv_off, st_off;
  int L, qs, kvs, cut;
};
template <typename Shape>
__device__ __forceinline__ HeadView head_view(const Shape& s, int b, int h, int D) {
  HeadView v;
  const int hkv = h / (s.H / s.Hkv);
  if (s.cu == nullptr) {
    v.L = s.N;
    v.cut = 0;
    v.qs = D;
    v.kvs = D;
    v.q_off = ((size_t)b * s.H + h) * (size_t)s.N * D;
    v.kv_off = ((size_t)b * s.Hkv + hkv) * (size_t)s.N * D;
    v.st_off = ((size_t)b * s.H + h) * (size_t)s.N;
  } else {
    // Clamped so that a malformed cu_seqlens can leave rows unwritten but can
    // never address memory outside [0, total) or past the grid's N rows.
    const int t0 = min(max(s.cu[b], 0), s.total);
    const int t1 = min(max(s.cu[b + 1], t0), s.total);
    v.L = min(t1 - t0, s.N);
    v.cut = (t1 - t0) > s.N;
    v.qs = s.H * D;
    v.kvs = s.Hkv * D;
    v.q_off = (size_t)t0 * s.H * D + (size_t)h * D;
    v.kv_off = (size_t)t0 * s.Hkv * D + (size_t)hkv * D;
    v.st_off = (size_t)h * s.total + t0;
  }
  return v;
}
// The view of query head h + j of the same batch entry, from the view of head
// h (query-side offsets only; the key/value fields are left as they are).
template <typename Shape>
__device__ __forceinline__ HeadView step_head(HeadView v, const Shape& s, int j, int D) {
  if (s.cu == nullptr) {
    v.q_off += (size_t)j * s.N * D;
    v.st_off += (size_t)j * s.N;
  } else {
    v.q_off += (size_t)j * D;
    v.st_off += (size_t)j * s.total;
  }
  return v;
}

// Key (or query) offset inside a 64-row tile of register r of C block kb, for
// a lane in half g, when the A rows of the product were read via perm_row().
__device__ __forceinline__ int crow(int kb, int r, int g) { return 32 * kb + 16 * (r >> 3) + 8 * g + (r & 7); }

// Linear block id -> (tile rank, batch entry, head) for a grid of R tile
// ranks per unit, units numbered head-major (u = h·B + b).  Blocks go
// round-robin over the 8 XCDs (XCD x runs the ids with id % 8 == x) and
// each XCD takes a contiguous range of units, so grouped heads (consecutive)
// and whole heads of a batch share that XCD's L2.  With up to 32 units per
// XCD the blocks go rank by rank across all of them: rank 0 (the caller's
// heaviest tile) of every unit first.  With more units (many sequences of a
// batch) they go in groups of G units, rank by rank within a group: G is
// about 64 blocks' worth of units, so the concurrently running blocks stream
// few units' key/value rows (L2 reuse) while each group still runs heaviest
// first; with grouped heads (group > 1) G also covers the B·group units among
// which every batch entry's query heads read the same key/value rows.
// unit_major (the forward): with up to 32 units per XCD but at least 64 ranks
// per unit, two units (or two groups of heads sharing key/value rows) at a
// time instead, rank by rank within them: the XCD's ~32 concurrent blocks
// then stream the key/value rows of two heads rather than of all of the
// XCD's heads, which cuts the HBM re-reads of a long causal forward by 40% at
// the same speed.  (One unit at a time cuts them by 56% but costs ~1%; with
// fewer ranks the causal imbalance at the end costs more than either.)
__device__ __forceinline__ void map_unit(int bid, int B, int H, int group, int& rank, int& b, int& h,
                                         bool unit_major = false) {
  const int BH = B * H;
  const bool split = (BH & 7) == 0;
  const int upx = split ? BH >> 3 : BH;  // units per XCD
  const int slot = split ? bid >> 3 : bid;
  const int base = split ? (bid & 7) * upx : 0;
  const int R = gridDim.x / BH;
  int u;
  if (upx <= 32 && !(unit_major && R >= 64)) {
    rank = slot / upx;
    u = base + slot % upx;
  } else {
    const int G = upx <= 32 ? min(upx, 2 * group) : min(upx, max((64 + R - 1) / R, group > 1 ? B * group : 1));
    const int grp = slot / (G * R), idx = slot % (G * R);
    const int gs = min(G, upx - grp * G);  // units in this group (the last may have fewer)
    rank = idx / gs;
    u = base + grp * G + idx % gs;
  }
  b = u % B;
  h = u / B;
}

// The same mapping for batches of several sequences whose ranks of a unit all
// read the start of the same key/value rows (a paged prefill: every query tile
// of a chunk streams the cached prefix first; a packed causal batch: every
// query tile streams the sequence from its first key).  When an XCD's range of
// the head-major numbering is whole key/value heads of every batch entry, its
// blocks go one (batch entry, key/value head) at a time: the `group` query
// heads x all ranks, heaviest rank first.  The XCD's ~32 concurrent blocks then
// read one prefix up to 32 ways; rank by rank, a chunked prefill of 8
// sequences read 8 prefixes 4 ways and hit L2 on 31% of its tile reads (93%
// this way).  Every XCD still holds a slice of every batch entry.  Other
// shapes fall back to map_unit.
__device__ __forceinline__ void map_unit_kv(int bid, int B, int H, int group, int& rank, int& b, int& h) {
  const int BH = B * H;
  const int upx = BH >> 3;
  if ((BH & 7) != 0 || upx % (B * group) != 0) {
    map_unit(bid, B, H, group, rank, b, h, true);
    return;
  }
  const int R = gridDim.x / BH;
  const int slot = bid >> 3;
  const int per = group * R;                  // blocks of one (batch entry, key/value head)
  const int k = slot / per, idx = slot % per;
  rank = idx / group;
  b = k % B;
  h = (bid & 7) * (upx / B) + (k / B) * group + idx % group;
}

// Compile-time loop: f(std::integral_constant<int, I>) for I = B .. E-1.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Matrix products written as single instructions so that each operand sits
// in the register file it is used from: blocks the VALU reads (scores) in
// VGPRs; blocks only the matrix unit touches (output and gradient
// accumulators, operands held for a whole pass) in AGPRs.  The compiler
// cannot see the latency of these instructions: a VALU read of their results
// that is not already separated by later pipeline slots is preceded by
// mfma_drain().
//   mfma_s0: s = a·b   mfma_s: s += a·b   (s in VGPRs, b in AGPRs)
//   mfma_o:  o += a·p                     (o in AGPRs)
__device__ __forceinline__ void mfma_s0(f32x16& s, const bf16x8& a, const bf16x8& q) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(a), "a"(q));
}
__device__ __forceinline__ void mfma_s(f32x16& s, const bf16x8& a, const bf16x8& q) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(a), "a"(q));
}
__device__ __forceinline__ void mfma_o(f32x16& o, const bf16x8& a, const bf16x8& p) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(a), "v"(p));
}
// The same on 16x16x32 products (result: 4 registers per lane); the _here
// forms are volatile, pinned in program order for software pipelines whose
// slots are laid out by hand.
__device__ __forceinline__ void mfma16_s0(f32x4& s, const bf16x8& a, const bf16x8& q) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(a), "a"(q));
}
__device__ __forceinline__ void mfma16_s(f32x4& s, const bf16x8& a, const bf16x8& q) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(a), "a"(q));
}
__device__ __forceinline__ void mfma16_s0_here(f32x4& s, const bf16x8& a, const bf16x8& q) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(a), "a"(q));
}
__device__ __forceinline__ void mfma16_s_here(f32x4& s, const bf16x8& a, const bf16x8& q) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(a), "a"(q));
}
__device__ __forceinline__ void mfma16_o_here(f32x4& o, const bf16x8& a, const bf16x8& p) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(a), "v"(p));
}
// More wait states than a 32x32x16 or 16x16x32 product needs before its result is read.
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

}  // namespace fa
