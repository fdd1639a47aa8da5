// Fused exact-attention forward for gfx950.
//
// One workgroup owns a tile of 256 queries of one (batch, head); each of its
// eight wavefronts owns 32 of those queries.  Key/value tiles of 64 tokens
// stream HBM -> LDS through direct buffer loads into a two-stage ring (K one
// tile ahead of V), and per tile a wave
//   1. computes Sᵀ = K·Qᵀ (64 keys x 32 queries) on bf16 MFMA, Q kept in
//      registers for the whole pass,
//   2. masks future keys (diagonal tiles only) and keys past N,
//   3. runs the online softmax: p = 2^(s·scale·log2e − m) against a running
//      reference max m that moves (rescaling the partial output and the
//      normaliser) only when the max grows by more than 2^8,
//   4. rounds p to bf16 and accumulates Oᵀ += Vᵀ·Pᵀ on MFMA, with Vᵀ read
//      transposed out of the row-major V tile (ds_read_b64_tr_b16).
// The scores of tile t+1 are computed on the matrix pipe while the VALU turns
// tile t into probabilities.  Holding Sᵀ (one query per lane) keeps every row
// reduction inside a lane plus one exchange with lane ^ 32, and makes the
// rescale of O a per-lane scalar.  Only O (bf16, round-to-nearest-even) and
// the natural-log logsumexp are written back; no score tile ever reaches
// device memory.
//
// Method: "Flash Attention 是什么：2026 最新原理、架构演进与实战详解"
// (ai.lansai.wang), 技术原理 › 核心工作机制 (tiling into on-chip memory and
// the online softmax) and 关键术语解析 §4 (the running max m and normaliser l
// updates); zwxr.cn §3.1 (rescale by the final normaliser once at the end).
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kBR = 256;  // queries per workgroup
constexpr int kBC = 64;   // keys per tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

// m = max(m, a, b) as one v_max3_f32 that stays where it is written: work
// scheduled into a pipeline slot must not be sunk out of it into the branch
// that consumes it.
__device__ __forceinline__ void max3_here(float& m, float a, float b) {
  asm volatile("v_max3_f32 %0, %0, %1, %2" : "+v"(m) : "v"(a), "v"(b));
}

// Pipeline slot of the fma of score value x (0 .. 63, pair x / 2) of a tile:
// the 64 values are spread evenly over slots 0 .. SPAN-1; the value's exp
// issues one slot later, the pair's pack and sum one slot after its second
// exp, and the running sum one slot after that.
template <int SPAN>
constexpr int fma_slot(int x) {
  return (x * SPAN) / 64;
}
// The value whose fma is in slot s (at most one: SPAN >= 64 makes fma_slot
// strictly increasing), or -1.
template <int SPAN>
constexpr int value_at_slot(int s) {
  static_assert(SPAN >= 64, "one fma per slot at most");
  for (int x = 0; x < 64; ++x)
    if (fma_slot<SPAN>(x) == s) return x;
  return -1;
}

// Rescale the output only when the running max grows by more than this many
// powers of two.  Between rescales p = 2^(s·scale·log2e − m) <= 2^8: the
// output, its normaliser and the logsumexp all use the same reference m, so
// the result is the same exact quantity (only rounding differs).
constexpr float kRescaleThreshold = 8.0f;
// The d = 128 forward's sum check: a row whose sum passes 2^20 is scaled back
// by a power of two; one whose sum reaches 2^40 (or is not a number) sends its
// workgroup through the exact-max loop instead.  A sum below 2^40 bounds every
// p, and each partial output by 2^40 times the largest |v|.
constexpr float kSumRescale = 1048576.0f;     // 2^20
constexpr float kSumLimit = 1099511627776.0f;  // 2^40

constexpr int kPage = 256;  // tokens per page of a paged key/value pool
// Slots between an LDS operand read and the product that consumes it.
constexpr int kLook = 2;

// bf16 bits of x rounded to nearest (ties to even) in one step from fp64:
// add half of the 45 dropped mantissa bits (minus one, plus the lowest kept
// bit) and clear them; the result is exact in fp32, whose top half it is.
__device__ __forceinline__ uint32_t bf16_rne_f64(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  u = (u + ((1ull << 44) - 1) + ((u >> 45) & 1)) & ~((1ull << 45) - 1);
  return __float_as_uint((float)__longlong_as_double((long long)u)) >> 16;
}

// Rotation of feature pairs (a, b) by (c, s), rounded to bf16: the exact
// rotation (a·c − b·s, a·s + b·c) rounded to nearest.  Computed in fp32,
// whose error is below e = 2^-21·(|a|+|b|)·(|c|+|s|); when the bf16 roundings
// of (x − e, y − e) and (x + e, y + e) agree (one packed pair each, compared
// as one word), every value in between (the exact one included) rounds the
// same way, and the lower pair is the result.  Otherwise (rare: a value
// within e of a rounding boundary) the lane recomputes its pairs in fp64,
// where the products of bf16 and fp32 values are exact and only the sum is
// rounded, and rounds that directly.  NP pairs at a time; out[j] holds pair
// j as (x in the low 16 bits, y in the high 16 bits).
template <int NP>
__device__ __forceinline__ void rotate_pairs(const float* a, const float* b, const float* c, const float* s,
                                             uint32_t* out) {
  bool bad = false;
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const float xr = __builtin_fmaf(a[j], c[j], -(b[j] * s[j]));
    const float yr = __builtin_fmaf(a[j], s[j], b[j] * c[j]);
    const float e =
        (__builtin_fabsf(a[j]) + __builtin_fabsf(b[j])) * (__builtin_fabsf(c[j]) + __builtin_fabsf(s[j])) * 0x1p-21f;
    out[j] = pack_bf16x2(xr - e, yr - e);
    bad = bad || (out[j] != pack_bf16x2(xr + e, yr + e));
  }
  if (bad) {
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const double ad = a[j], bd = b[j], cd = c[j], sd = s[j];
      out[j] = bf16_rne_f64(ad * cd - bd * sd) | (bf16_rne_f64(ad * sd + bd * cd) << 16);
    }
  }
}

// Rotate the feature pairs (x[j], y[j]) of 8 bf16 values each by the angles
// whose cosines / sines are c[j], s[j].
// Two pairs at a time (one word of x, one of y), which keeps the live
// registers within the kernel's budget.
__device__ __forceinline__ void rotate8(bf16x8& x, bf16x8& y, const float* c, const float* s) {
  u32x4 wx, wy;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a[2] = {(float)x[2 * k], (float)x[2 * k + 1]};
    const float b[2] = {(float)y[2 * k], (float)y[2 * k + 1]};
    uint32_t r[2];
    rotate_pairs<2>(a, b, c + 2 * k, s + 2 * k, r);
    wx[k] = (r[0] & 0xffffu) | (r[1] << 16);
    wy[k] = (r[0] >> 16) | (r[1] & 0xffff0000u);
  }
  x = __builtin_bit_cast(bf16x8, wx);
  y = __builtin_bit_cast(bf16x8, wy);
}
// Same for the interleaved pairing: pairs (x[2j], x[2j+1]), angles c[j], s[j].
__device__ __forceinline__ void rotate8_interleaved(bf16x8& x, const float* c, const float* s) {
  u32x4 w;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float a[2] = {(float)x[4 * k], (float)x[4 * k + 2]};
    const float b[2] = {(float)x[4 * k + 1], (float)x[4 * k + 3]};
    uint32_t r[2];
    rotate_pairs<2>(a, b, c + 2 * k, s + 2 * k, r);
    w[2 * k] = r[0];
    w[2 * k + 1] = r[1];
  }
  x = __builtin_bit_cast(bf16x8, w);
}
template <int N>
__device__ __forceinline__ void load_f32(float* dst, const float* src) {
#pragma unroll
  for (int j = 0; j < N; j += 4) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(src + j);
    dst[j] = v[0];
    dst[j + 1] = v[1];
    dst[j + 2] = v[2];
    dst[j + 3] = v[3];
  }
}

template <int D, bool CAUSAL, bool PAGED, bool ROPE>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, AttnShape shape, PagedKV pkv, RopeArgs rope,
    float scale_log2) {
  constexpr int KSTEPS = D / 16;  // MFMA k-steps over the head dim
  constexpr int DBLK = D / 32;    // 32-row output blocks over the head dim
  constexpr int TILE = kTileRows * D;
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int ROWS_PER_DMA = 64 / CPR;      // rows per 1 KiB wavefront load
  constexpr int DMA_PER_WAVE = kTileRows / ROWS_PER_DMA / kWaves;
  // K ring (2 tiles) and V ring (2 tiles), all row-major [64][D].  K runs one
  // tile ahead of V: while tile t is consumed, K(t+1) is already resident.
  // Each slot is its own LDS object and the loop below names slots at
  // compile time, so the compiler can tell that reads of one slot do not
  // depend on direct-to-LDS loads still in flight into another.
  __shared__ __attribute__((aligned(1024))) bf16 kbuf0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 kbuf1[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 vbuf0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 vbuf1[TILE];
  __shared__ int ptab[PAGED ? kMaxPrefillPages : 1];  // this sequence's pool pages
  // Rotary tables of the K tiles in the ring (one object per tile parity, as
  // the K slots): the cosines, then the sines, of the tile's 64 positions,
  // loaded with the K tile so that the rotation reads them from LDS.
  constexpr int RT = (ROPE && !PAGED) ? kTileRows * (D / 2) : 1;
  __shared__ __attribute__((aligned(1024))) float rtab0[2 * RT];
  __shared__ __attribute__((aligned(1024))) float rtab1[2 * RT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, n = lane & 31;
  int rank, bi, hi;
  map_unit(blockIdx.x, shape.B, shape.H, shape.H / shape.Hkv, rank, bi, hi, true);
  const HeadView hv = head_view(shape, bi, hi, D);
  const int N = hv.L;  // this sequence's queries
  const int nqb = (N + kBR - 1) / kBR;
  if (rank >= nqb) return;  // a shorter sequence of a packed batch: no tile of this rank
  const int qb = CAUSAL ? nqb - 1 - rank : rank;  // causal: the last query tiles see the most keys
  const int q0 = qb * kBR;
  // Keys of this sequence and the causal offset: query q sees keys 0 .. q + off.
  int Nk = N, off = 0;
  const int kvs = PAGED ? shape.Hkv * D : hv.kvs;  // elements between consecutive key rows
  const int hkv = hi / (shape.H / shape.Hkv);
  if constexpr (PAGED) {
    Nk = min(max(pkv.seq_lens[bi], 0), pkv.max_blocks * kPage);
    off = Nk - N;
    const int np = (Nk + kPage - 1) / kPage;
    for (int i = tid; i < np; i += kThreads)
      ptab[i] = min(max(pkv.block_table[(size_t)bi * pkv.max_blocks + i], 0), pkv.num_pages - 1);
    __syncthreads();
  }

  const auto rq = make_rsrc(Q + hv.q_off, (uint32_t)N * hv.qs * 2);
  const auto rk = make_rsrc(K + hv.kv_off, (uint32_t)N * hv.kvs * 2);
  const auto rv = make_rsrc(V + hv.kv_off, (uint32_t)N * hv.kvs * 2);
  // Paged: key tile t (64 rows) is rows (t % 4)·64.. of pool page ptab[t / 4]; its
  // descriptor ends at the sequence's last key, so later slots are never fetched.
  auto page_rsrc = [&](int t, int half) {
    // the page id is the same for every lane (one LDS address): keep the
    // descriptor in scalar registers
    const int page = __builtin_amdgcn_readfirstlane(ptab[t >> 2]);
    const bf16* base = static_cast<const bf16*>(pkv.pool) +
                       ((size_t)page * 2 * kPage + (size_t)half * kPage + (t & 3) * kTileRows) * kvs +
                       (size_t)hkv * D;
    return make_rsrc(base, (uint32_t)min(kTileRows, Nk - t * kTileRows) * kvs * 2);
  };
  const int qw = q0 + wave * 32;
  const int qrow = qw + n;  // this lane's query

  // Qᵀ as the B operand: lane (g, n) holds Q[qrow][16kk + 8g .. +7] (zeros past N).
  bf16x8 qreg[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk)
    qreg[kk] = __builtin_bit_cast(bf16x8, buf_load16(rq, (uint32_t)qrow * (hv.qs * 2) + (16 * kk + 8 * g) * 2));

  // Rotary embedding of this lane's query (position qrow + off; rows past N
  // take any valid table row: their outputs are never written).
  if constexpr (ROPE) {
    const int pos = min(max(qrow + off, 0), rope.rows - 1);
    const float* cr = rope.cos + (size_t)pos * (D / 2);
    const float* sr = rope.sin + (size_t)pos * (D / 2);
    if (!rope.interleaved) {
#pragma unroll
      for (int kk = 0; kk < KSTEPS / 2; ++kk) {  // features 16kk+8g.. pair with the same + D/2 (chunk kk + KSTEPS/2)
        float c[8], sn[8];
        load_f32<8>(c, cr + 16 * kk + 8 * g);
        load_f32<8>(sn, sr + 16 * kk + 8 * g);
        rotate8(qreg[kk], qreg[kk + KSTEPS / 2], c, sn);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {  // pairs (2i, 2i+1) inside the chunk, i from 8kk + 4g
        float c[4], sn[4];
        load_f32<4>(c, cr + 8 * kk + 4 * g);
        load_f32<4>(sn, sr + 8 * kk + 4 * g);
        rotate8_interleaved(qreg[kk], c, sn);
      }
    }
  }
  // Rotary embedding of a resident K tile (rows k0.., positions k0 + r), in
  // place in LDS: once per workgroup and tile, every thread one item.  The
  // tables of the tile's positions are already in LDS (tab: cosines, then
  // sines; rows past the table read as zero, and so do those K rows).
  auto rope_k = [&](bf16* ks, const float* tab) {
    if constexpr (ROPE && !PAGED) {
      if (!rope.interleaved) {
        constexpr int PAIRS = CPR / 2;  // chunk c pairs with chunk c + CPR/2
        for (int w = tid; w < kTileRows * PAIRS; w += kThreads) {
          const int r = w / PAIRS, c = w % PAIRS;
          bf16x8* px = reinterpret_cast<bf16x8*>(ks + r * D + ((c ^ rm_swz<D>(r)) << 3));
          bf16x8* py = reinterpret_cast<bf16x8*>(ks + r * D + (((c + PAIRS) ^ rm_swz<D>(r)) << 3));
          float cs[8], sn[8];
          load_f32<8>(cs, tab + r * (D / 2) + 8 * c);
          load_f32<8>(sn, tab + RT + r * (D / 2) + 8 * c);
          bf16x8 x = *px, y = *py;
          rotate8(x, y, cs, sn);
          *px = x;
          *py = y;
        }
      } else {
        for (int w = tid; w < kTileRows * CPR; w += kThreads) {
          const int r = w / CPR, c = w % CPR;
          bf16x8* px = reinterpret_cast<bf16x8*>(ks + r * D + ((c ^ rm_swz<D>(r)) << 3));
          float cs[4], sn[4];
          load_f32<4>(cs, tab + r * (D / 2) + 4 * c);
          load_f32<4>(sn, tab + RT + r * (D / 2) + 4 * c);
          bf16x8 x = *px;
          rotate8_interleaved(x, cs, sn);
          *px = x;
        }
      }
      __syncthreads();
    }
  };

  // Direct-to-LDS loads: wave w fills 1 KiB blocks w*DMA_PER_WAVE.. of a tile;
  // lane l writes physical chunk l % CPR of row l / CPR of its block, fetching
  // the logical chunk that the tile's swizzle puts there.
  const int dma_row = lane / CPR, dma_pc = lane % CPR;
  uint32_t kdma[DMA_PER_WAVE], vdma[DMA_PER_WAVE];
#pragma unroll
  for (int i = 0; i < DMA_PER_WAVE; ++i) {
    const int row = (wave * DMA_PER_WAVE + i) * ROWS_PER_DMA + dma_row;
    kdma[i] = (uint32_t)row * (kvs * 2) + ((dma_pc ^ rm_swz<D>(row)) << 4);
    vdma[i] = (uint32_t)row * (kvs * 2) + ((dma_pc ^ v_swz<D>(row)) << 4);
  }
  // Tile t of K (or V) into the given slot (t's parity: the caller names it).
  auto issue_k = [&](bf16* slot, int t) {
    if constexpr (PAGED) {
      const auto r = page_rsrc(t, 0);
#pragma unroll
      for (int i = 0; i < DMA_PER_WAVE; ++i) lds_dma16(r, slot + (wave * DMA_PER_WAVE + i) * 512, kdma[i]);
    } else {
#pragma unroll
      for (int i = 0; i < DMA_PER_WAVE; ++i)
        lds_dma16(rk, slot + (wave * DMA_PER_WAVE + i) * 512, kdma[i] + (uint32_t)t * (64 * kvs * 2));
    }
  };
  auto issue_v = [&](bf16* slot, int t) {
    if constexpr (PAGED) {
      const auto r = page_rsrc(t, 1);
#pragma unroll
      for (int i = 0; i < DMA_PER_WAVE; ++i) lds_dma16(r, slot + (wave * DMA_PER_WAVE + i) * 512, vdma[i]);
    } else {
#pragma unroll
      for (int i = 0; i < DMA_PER_WAVE; ++i)
        lds_dma16(rv, slot + (wave * DMA_PER_WAVE + i) * 512, vdma[i] + (uint32_t)t * (64 * kvs * 2));
    }
  };

  // The rotary tables of K tile t into a table slot: 64 table rows of D/2
  // fp32 each (one contiguous block per table) as 1 KiB direct-to-LDS loads,
  // lane l writing bytes 16l..16l+15 of its block; rows past the tables'
  // end read as zero.
  auto issue_tab = [&](float* tab, int t) {
    if constexpr (ROPE && !PAGED) {
      constexpr int BYTES = kTileRows * (D / 2) * 4;
      constexpr int NB = BYTES / 1024, PER = NB / kWaves;
      static_assert(PER >= 1 && NB % kWaves == 0, "table blocks split evenly over the wavefronts");
      const uint32_t tbytes = (uint32_t)max(rope.rows, 0) * (uint32_t)(D / 2) * 4u;
      const auto rc = make_rsrc(rope.cos, tbytes), rs = make_rsrc(rope.sin, tbytes);
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int blk = wave * PER + i;
        const uint32_t off = (uint32_t)t * (uint32_t)BYTES + (uint32_t)blk * 1024u + 16u * (uint32_t)lane;
        lds_dma16(rc, tab + blk * 256, off);
        lds_dma16(rs, tab + RT + blk * 256, off);
      }
    }
  };

  // Per-lane LDS element offsets of the operand reads (loop invariant).
  int koff[KSTEPS];  // K rows perm_row(n) (+32 for the second block), chunk 2kk+g
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) koff[kk] = perm_row(n) * D + (((2 * kk + g) ^ (n & (CPR - 1))) << 3);
  const int G = lane >> 4, j16 = lane & 15;
  int voff[DBLK];    // V read transposed: rows 8(G>>1) + j/4 (+16kk + 4c), column 32b + 16(G&1) + 4(j%4)
#pragma unroll
  for (int b = 0; b < DBLK; ++b) {
    const int row = 8 * (G >> 1) + (j16 >> 2);
    const int col = 32 * b + 16 * (G & 1) + 4 * (j16 & 3);
    voff[b] = row * D + (((col >> 3) ^ v_swz<D>(row)) << 3) + (col & 7);
  }

  // Sᵀ = K Qᵀ for one 64-key tile (16 LDS reads + 16 MFMA).
  auto scores = [&](const bf16* ks, f32x16* s) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = mfma32(*reinterpret_cast<const bf16x8*>(ks + kb * 32 * D + koff[0]), qreg[0], f32x16{});
#pragma unroll
      for (int kk = 1; kk < KSTEPS; ++kk)
        s[kb] = mfma32(*reinterpret_cast<const bf16x8*>(ks + kb * 32 * D + koff[kk]), qreg[kk], s[kb]);
    }
  };
  // Future keys (causal diagonal) and keys past the sequence's last get -inf.
  auto mask = [&](int k0, f32x16* s) {
    if ((CAUSAL && k0 + kBC - 1 > qw + off) || (k0 + kBC > Nk)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + crow(kb, r, g);
          const bool dead = (key >= Nk) || (CAUSAL && key > qrow + off);
          s[kb][r] = dead ? kNegInf : s[kb][r];
        }
    }
  };
  auto tile_max = [&](const f32x16* s) {
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    return xhalf_max(mx) * scale_log2;
  };

  f32x16 oacc[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;
  float m_run = kNegInf;  // reference max of s·scale·log2e (lags the true max by < 2^threshold)
  float l_run = 0.f;      // this lane's part of the normaliser

  const int kv_end = CAUSAL ? min(Nk, max(q0 + kBR + off, 0)) : Nk;
  const int ntiles = (kv_end + kBC - 1) / kBC;
  // tiles this wave needs (causal: up to its last query's last key; none past the keys)
  const int wlast = min(qw + 31, N - 1) + off;  // causal: this wave's last visible key
  const int wnt = (qw >= N) ? 0 : (CAUSAL ? (wlast < 0 ? 0 : min(ntiles, wlast / kBC + 1)) : ntiles);

  if (ntiles > 0) issue_k(kbuf0, 0);
  if (ntiles > 0) issue_tab(rtab0, 0);
  if (ntiles > 1) issue_k(kbuf1, 1);
  if (ntiles > 1) issue_tab(rtab1, 1);
  if (ntiles > 0) issue_v(vbuf0, 0);
  wait_vm_all();
  __syncthreads();
  if (ntiles > 0) rope_k(kbuf0, rtab0);
  f32x16 sa[2], sb[2];
  if (wnt > 0) {
    scores(kbuf0, sa);
    mask(0, sa);
    m_run = tile_max(sa);  // first tile: nothing to rescale yet
  }

  // One tile: P(t) from S(t) = sc, while S(t+1) = sn is computed on the matrix
  // pipe; then O += V(t)ᵀ P(t); then S(t+1) is masked and its max checked.
  // One tile as a fixed software pipeline of NS + NP fenced slots, one matrix
  // product each.  Slots 0 .. NS-1 compute S(t+1) = K(t+1)·Qᵀ (on a wave's last
  // tile they read a stale K tile and are dropped); slots NS .. NS+NP-1
  // accumulate Oᵀ += Vᵀ·Pᵀ, key chunk by key chunk.  The VALU work rides
  // along: the 16 pairs of S(t) scores become bf16 probabilities in the first
  // slots (pair pi by slot pi·SPAN/16, before the product that first needs
  // its chunk), and the last slots take the max of S(t+1).  A diagonal or
  // tail tile (maskn) is masked and its max retaken after the slots.  Every
  // LDS operand is read LOOK slots ahead of its product; the fences keep the
  // compiler from undoing the order.
  constexpr int LOOK = kLook;
  constexpr int NS = 2 * KSTEPS;     // products of S(t+1)
  constexpr int NP = 4 * DBLK;       // products of Oᵀ += Vᵀ·Pᵀ
  constexpr int NT = NS + NP;
  constexpr int SPAN = NS + 3 * DBLK - 2;
  constexpr int MAX0 = NS + 2;       // first slot that reads S(t+1)
  auto tile_slots = [&](bool maskn, int t, f32x16* sc, f32x16* sn, const bf16* kn, const bf16* vs) {
    auto kread = [&](int i) {  // K operand of S product i: key block i / KSTEPS, k-step i % KSTEPS
      return *reinterpret_cast<const bf16x8*>(kn + (i / KSTEPS) * 32 * D + koff[i % KSTEPS]);
    };
    auto vread = [&](int j) {  // Vᵀ operand of P·V product j: key chunk j / DBLK, d block j % DBLK
      const bf16* base = vs + voff[j % DBLK] + 16 * (j / DBLK) * D;
      const bf16x4 lo = lds_read_tr4(base);
      const bf16x4 hi = lds_read_tr4(base + 4 * D);
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    const float m_use = (m_run == kNegInf) ? 0.f : m_run;
    bf16x8 op[LOOK + 1];
    u32x4 pw[4];  // P(t) as packed bf16 pairs: pw[2kb + h] holds keys 32kb + 16h ..
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < LOOK; ++i) op[i] = kread(i);
#pragma unroll
    for (int sl = 0; sl < NT; ++sl) {
      // operand read for the product LOOK slots ahead
      const int ahead = sl + LOOK;
      if (ahead < NS)
        op[ahead % (LOOK + 1)] = kread(ahead);
      else if (ahead < NT)
        op[ahead % (LOOK + 1)] = vread(ahead - NS);
      // this slot's product
      if (sl < NS) {
        const int kb = sl / KSTEPS, kk = sl % KSTEPS;
        sn[kb] = mfma32(op[sl % (LOOK + 1)], qreg[kk], kk == 0 ? f32x16{} : sn[kb]);
      } else {
        const int j = sl - NS;
        const int kk = j / DBLK, b = j % DBLK;
        oacc[b] = mfma32(op[sl % (LOOK + 1)], __builtin_bit_cast(bf16x8, pw[kk]), oacc[b]);
      }
      // probabilities of S(t) for the pairs scheduled here
#pragma unroll
      for (int pi = 0; pi < 16; ++pi) {
        if ((pi * SPAN) / 16 != sl) continue;
        const int pkb = pi / 8, r = 2 * (pi % 8);
        const float p0 = exp2_fast(__builtin_fmaf(sc[pkb][r], scale_log2, -m_use));
        const float p1 = exp2_fast(__builtin_fmaf(sc[pkb][r + 1], scale_log2, -m_use));
        pw[2 * pkb + r / 8][(r % 8) / 2] = pack_bf16x2(p0, p1);
        l_run += p0 + p1;  // fp32 sum of the unrounded p: the logsumexp needs it exact
      }
      // max of S(t+1) for the values scheduled here
#pragma unroll
      for (int v = 0; v < 32; v += 2) {
        if (MAX0 + (v * (NT - MAX0)) / 32 != sl) continue;
        max3_here(mx, sn[v / 16][v % 16], sn[v / 16][v % 16 + 1]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // Move the reference max for tile t+1 if it grew too far (O now holds tile t).
    if (t + 1 < wnt) {
      if (maskn) {
        mask((t + 1) * kBC, sn);
        mx = kNegInf;
#pragma unroll
        for (int v = 0; v < 32; ++v) mx = fmaxf(mx, sn[v / 16][v % 16]);
      }
      mx = xhalf_max(mx) * scale_log2;
      if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleThreshold)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = exp2_fast(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int b = 0; b < DBLK; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;
        m_run = m_new;
      }
    }
  };

  // kc / vc: the slots of tile t (parity of t); kn / vn: the other ones.
  auto step = [&](int t, f32x16* sc, f32x16* sn, bf16* kc, bf16* kn, bf16* vc, bf16* vn, float* tc, float* tn) {
    const int k0 = t * kBC;
    wait_vm_all();
    __syncthreads();  // K(t+1) and V(t) resident for every wave; tile t-1 fully consumed
    if (t + 2 < ntiles) issue_k(kc, t + 2);
    if (t + 2 < ntiles) issue_tab(tc, t + 2);
    if (t + 1 < ntiles) issue_v(vn, t + 1);
    if (k0 + kBC > Nk) {  // tail tile: V rows past the last key must read as zero, whatever the loads left
      const int first = Nk - k0;
      for (int idx = tid; idx < (kBC - first) * CPR; idx += kThreads) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(vc + (first + idx / CPR) * D + (idx % CPR) * 8) = z;
      }
      __syncthreads();
    }
    if (t + 1 < ntiles) rope_k(kn, tn);
    if (t >= wnt) return;
    const int k0n = k0 + kBC;
    tile_slots((CAUSAL && k0n + kBC - 1 > qw + off) || (k0n + kBC > Nk), t, sc, sn, kn, vc);
  };

  for (int t = 0; t < ntiles; t += 2) {  // unrolled by two so S(t) and S(t+1) swap registers
    step(t, sa, sb, kbuf0, kbuf1, vbuf0, vbuf1, rtab0, rtab1);
    if (t + 1 < ntiles) step(t + 1, sb, sa, kbuf1, kbuf0, vbuf1, vbuf0, rtab1, rtab0);
  }

  if (qw >= N || qrow >= N) return;
  const float l_tot = xhalf_sum(l_run);
  // A query that sees no key (paged causal prefill with fewer keys than queries
  // before it) has an empty softmax: O = 0, LSE = -inf.
  const float inv = hv.cut ? kNaN : (l_tot > 0.f ? 1.f / l_tot : 0.f);
  bf16* Orow = O + hv.q_off + (size_t)qrow * hv.qs;
#pragma unroll
  for (int b = 0; b < DBLK; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x2 w;
      w[0] = pack_bf16x2(oacc[b][4 * i + 0] * inv, oacc[b][4 * i + 1] * inv);
      w[1] = pack_bf16x2(oacc[b][4 * i + 2] * inv, oacc[b][4 * i + 3] * inv);
      *reinterpret_cast<u32x2*>(Orow + 32 * b + 8 * i + 4 * g) = w;
    }
  if (LSE != nullptr && g == 0)
    LSE[hv.st_off + qrow] = hv.cut ? kNaN : (l_tot > 0.f ? (m_run + log2_fast(l_tot)) * kLn2 : kNegInf);
}

// The same forward with 64 queries per wavefront, for d = 128 with K/V laid
// out like the queries (dense, grouped heads, packed batches) or read
// through a page table (paged prefill): four wavefronts per workgroup, one
// per SIMD, on 16x16x32 products.  Under the board's power limit a
// 16x16x32 product costs less energy per FLOP than a 32x32x16 one (it reads
// and writes a quarter of the accumulator registers for half the work), so
// the clock the limit allows is higher.  Each K and Vᵀ operand read from LDS
// feeds four products (query blocks j = 0..3); the output accumulators and
// Qᵀ live in accumulation registers.
//
// Register layout of a 16x16x32 product (lane l, G = l / 16, i = l % 16):
// the A operand holds row i, k = 8G .. 8G+7; the B operand column i, the
// same k; the result holds column i, rows 4G .. 4G+3.  Sᵀ block (kb, j) is
// keys 16kb.. (rows) by queries 16j.. (columns): lane l holds query
// qw + 16j + i against keys 16kb + 4G + r, r = 0..3.  Those four keys of
// blocks 2c and 2c+1 are the eight k-values of the Pᵀ operand of key chunk
// c (32 keys), and the Vᵀ operand reads the same eight keys (4G.. and
// 16 + 4G.. of the chunk) with two transposed reads, so P needs no shuffle.
template <bool CAUSAL, bool PAGED>
__global__ __launch_bounds__(256, 1) void fwd_w64_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                                                         const bf16* __restrict__ V, bf16* __restrict__ O,
                                                         float* __restrict__ LSE, AttnShape shape, PagedKV pkv,
                                                         float scale_log2) {
  constexpr int D = 128;
  constexpr int KC = D / 32;   // 32-feature k-steps of Sᵀ = K·Qᵀ
  constexpr int QB = 4;        // 16-query blocks of a wavefront
  constexpr int KB = 4;        // 16-key blocks of a tile
  constexpr int DB = D / 16;   // 16-feature blocks of Oᵀ
  constexpr int TILE = kTileRows * D;
  constexpr int CPR = D / 8;
  constexpr int WAVES = 4;
  constexpr int THREADS = 64 * WAVES;
  constexpr int ROWS_PER_DMA = 64 / CPR;
  constexpr int DMA_PER_WAVE = kTileRows / ROWS_PER_DMA / WAVES;
  static_assert(ROWS_PER_DMA == 4 && DMA_PER_WAVE == 4, "tile loads: 4 rows per load, 4 loads per wavefront");
  __shared__ __attribute__((aligned(1024))) bf16 kbuf0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 kbuf1[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 vbuf0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 vbuf1[TILE];
  __shared__ int ptab[PAGED ? kMaxPrefillPages : 1];  // this sequence's pool pages
  __shared__ __attribute__((aligned(16))) float rsc[THREADS * 4];  // 16 bytes per lane: output rescale staging

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = lane >> 4, i16 = lane & 15;
  auto* rsc_lane = (__attribute__((address_space(3))) float*)(rsc + 4 * tid);
  int rank, bi, hi;
  if (PAGED || shape.cu != nullptr)
    map_unit_kv(blockIdx.x, shape.B, shape.H, shape.H / shape.Hkv, rank, bi, hi);
  else
    map_unit(blockIdx.x, shape.B, shape.H, shape.H / shape.Hkv, rank, bi, hi, true);
  const HeadView hv = head_view(shape, bi, hi, D);
  const int N = hv.L;
  const int nqb = (N + kBR - 1) / kBR;
  if (rank >= nqb) return;
  const int qb = CAUSAL ? nqb - 1 - rank : rank;
  const int q0 = qb * kBR;
  // Keys of this sequence and the causal offset: query q sees keys 0 .. q + off.
  int Nk = N, off = 0;
  const int kvs = PAGED ? shape.Hkv * D : hv.kvs;  // elements between consecutive key rows
  const int hkv = hi / (shape.H / shape.Hkv);
  if constexpr (PAGED) {
    Nk = min(max(pkv.seq_lens[bi], 0), pkv.max_blocks * kPage);
    off = Nk - N;
    const int np = (Nk + kPage - 1) / kPage;
    for (int i = tid; i < np; i += THREADS)
      ptab[i] = min(max(pkv.block_table[(size_t)bi * pkv.max_blocks + i], 0), pkv.num_pages - 1);
    __syncthreads();
  }
  const auto rq = make_rsrc(Q + hv.q_off, (uint32_t)N * hv.qs * 2);
  const auto rk = make_rsrc(K + hv.kv_off, (uint32_t)N * hv.kvs * 2);
  const auto rv = make_rsrc(V + hv.kv_off, (uint32_t)N * hv.kvs * 2);
  // Paged: key tile t (64 rows) is rows (t % 4)·64.. of pool page ptab[t / 4]
  // (K half 0, V half 1); the descriptor ends at the sequence's last key, so
  // later slots are never fetched.  Unpaged: the whole head, offset by the tile.
  auto tile_rsrc = [&](int t, int half) {
    if constexpr (PAGED) {
      const int page = __builtin_amdgcn_readfirstlane(ptab[t >> 2]);
      const bf16* base = K + ((size_t)page * 2 * kPage + (size_t)half * kPage + (t & 3) * kTileRows) * kvs +
                         (size_t)hkv * D;
      return make_rsrc(base, (uint32_t)max(min(kTileRows, Nk - t * kTileRows), 0) * kvs * 2);
    } else {
      return half ? rv : rk;
    }
  };
  // Byte offset of tile t inside tile_rsrc(t, ·).
  auto tile_base = [&](int t) { return PAGED ? 0u : (uint32_t)t * (uint32_t)(64 * kvs * 2); };
  const int qw = q0 + wave * 64;  // this wave's first query; query block j holds qw + 16j ..

  // Qᵀ as the B operand of every query block (zeros past N).
  bf16x8 qreg[QB][KC];
#pragma unroll
  for (int j = 0; j < QB; ++j)
#pragma unroll
    for (int kk = 0; kk < KC; ++kk)
      qreg[j][kk] = __builtin_bit_cast(
          bf16x8, buf_load16(rq, (uint32_t)(qw + 16 * j + i16) * (hv.qs * 2) + (32 * kk + 8 * G) * 2));

  // Tile layout in LDS: row r of a tile at r·D; its 16-byte chunk c at
  // position c ^ (r % 16) (K) or c ^ (2r % 16) (V).  A K operand read (16
  // lanes: 16 rows, one chunk each) then covers all 16 chunk positions, and a
  // transposed V read (32 lanes: 8 consecutive rows x 2 chunks) 16 distinct
  // positions, so neither pattern has bank conflicts.  Direct-to-LDS loads
  // write lane l's 16 bytes at position l % 16 of row l / 16 of their
  // 4-row block, so each lane fetches the chunk that belongs there:
  // row r = 16·wave + 4i + G fetches chunk i16 ^ swizzle(r).
  const uint32_t drow = (uint32_t)(16 * wave + G) * (uint32_t)(kvs * 2);
  auto issue_k1 = [&](bf16* slot, __amdgpu_buffer_rsrc_t r, uint32_t tbase, int i) {
    const uint32_t ch = (uint32_t)(i16 ^ ((4 * i + G) & 15)) << 4;
    lds_dma16(r, slot + (wave * DMA_PER_WAVE + i) * 512, drow + ch + (tbase + (uint32_t)(4 * i * kvs * 2)));
  };
  auto issue_v1 = [&](bf16* slot, __amdgpu_buffer_rsrc_t r, uint32_t tbase, int i) {
    const uint32_t ch = (uint32_t)(i16 ^ ((8 * i + 2 * G) & 15)) << 4;
    lds_dma16(r, slot + (wave * DMA_PER_WAVE + i) * 512, drow + ch + (tbase + (uint32_t)(4 * i * kvs * 2)));
  };
  auto issue_k = [&](bf16* slot, int t) {
    const auto r = tile_rsrc(t, 0);
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) issue_k1(slot, r, tile_base(t), i);
  };
  auto issue_v = [&](bf16* slot, int t) {
    const auto r = tile_rsrc(t, 1);
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) issue_v1(slot, r, tile_base(t), i);
  };

  // LDS operand offsets (elements).  K block kb, k-step kk: row 16kb + i16,
  // chunk 4kk + G at position (4kk + G) ^ i16 = 4kk ^ (G ^ i16).  Vᵀ block db,
  // key chunk c, half h: lanes address row 32c + 16h + vr (vr = 4G + i16/4),
  // columns 16db + 4(i16 % 4).. (chunk 2db + (i16 % 4)/2, at position
  // (2db + x) ^ 2(vr % 8) = 2(db ^ (vr % 8)) + x).
  const int kbase = i16 * D;
  const int kx = (G ^ i16) << 3;
  auto koff = [&](int kb, int kk) { return kb * 16 * D + kbase + (kx ^ (kk << 5)); };
  const int vr = 4 * G + (i16 >> 2);
  const int vbase = vr * D + (((i16 & 3) >> 1) << 3) + 4 * (i16 & 1);
  const int vx = (vr & 7) << 4;
  auto voff = [&](int db, int c, int h) { return (32 * c + 16 * h) * D + vbase + (vx ^ (db << 4)); };

  // s[4kb + j]: Sᵀ block of keys 16kb.., queries 16j.. (register r: key 16kb + 4G + r, query 16j + i16).
  auto mask = [&](int k0, f32x4* s) {
    if ((CAUSAL && k0 + kBC - 1 > qw + off) || (k0 + kBC > Nk)) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int j = 0; j < QB; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = k0 + 16 * kb + 4 * G + r;
            const bool dead = (key >= Nk) || (CAUSAL && key > qw + 16 * j + i16 + off);
            s[4 * kb + j][r] = dead ? kNegInf : s[4 * kb + j][r];
          }
    }
  };
  // Max over the four lanes that share a query (l, l ^ 16, l ^ 32, l ^ 48).
  auto quad_max = [](float x) {
    const float y = xhalf_max(x);
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  };
  auto quad_sum = [](float x) {
    const float y = xhalf_sum(x);
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  };

  f32x4 oacc[DB][QB];
  // m_run: reference of s·scale·log2e of each query block, the same in the
  // four lanes of a query; l_run: this lane's part of the row sum.
  float m_run[QB], l_run[QB];

  const int kv_end = CAUSAL ? max(min(Nk, q0 + kBR + off), 0) : Nk;
  const int ntiles = (kv_end + kBC - 1) / kBC;
  const int wlast = min(qw + 63, N - 1) + off;  // the wave's last visible key (causal)
  const int wnt = (qw >= N) ? 0 : (CAUSAL ? (wlast < 0 ? 0 : min(ntiles, wlast / kBC + 1)) : ntiles);

  // Output block j of this lane's query times alpha.  Each accumulator block
  // goes out of the accumulation registers and back through this lane's own
  // 16 bytes of LDS, so the compiler never holds the output blocks anywhere
  // but in those registers.
  auto scale_out = [&](int j, float alpha) {
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      f32x4 x;
      asm volatile("ds_write_b128 %1, %2\n\ts_waitcnt lgkmcnt(0)\n\tds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                   : "=&v"(x)
                   : "v"(rsc_lane), "a"(oacc[b][j])
                   : "memory");
      x = x * alpha;
      asm volatile("ds_write_b128 %1, %2\n\ts_waitcnt lgkmcnt(0)\n\tds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                   : "=&a"(oacc[b][j])
                   : "v"(rsc_lane), "v"(x)
                   : "memory");
    }
  };

  // One tile: 128 product slots.  Slots 0..63 compute Sᵀ(t+1), one K operand
  // (block kb, k-step kk) per four slots, one query block per slot; slots
  // 64..127 accumulate Oᵀ += Vᵀ·Pᵀ(t), one Vᵀ operand (key chunk c, block db)
  // per four slots.  Every LDS operand is read three operands (twelve
  // products) ahead of its first product.
  constexpr int LOOK = 3;
  constexpr int NSL = 128;
  // Softmax of S(t): value x (0..63, pair x / 2) has its fma in slot
  // fma_slot<PSPAN>(x), its exp one slot later; the pair's pack and sum one
  // slot after its second exp, the row sum one after that.  Pairs go in the
  // order their Pᵀ operands are used: key chunk c, query block j, key block
  // 2c + h, register pair w (the last Pᵀ operand is packed by slot 92, five
  // slots before its first product).
  // Two ways to keep p bounded (EXACT below):
  //  * EXACT: the max of S(t+1), two scores per v_max3, spread over slots
  //    MAX0 .. MAX0 + MAXN - 1 of the output half, where every block of
  //    S(t+1) is complete; the reference moves (rescaling output and
  //    normaliser) when that max exceeds it by kRescaleThreshold.
  //  * sum check: no max at all.  The reference is the first tile's row max;
  //    after each tile a row whose sum exceeds kSumRescale has output and sum
  //    scaled by an exact power of two 2^-e and e added to its reference.  p
  //    never exceeds the row sum, so a sum below kSumLimit bounds every p and
  //    every partial output; a tile that lifts a sum past it (a jump of the
  //    scores by more than ~20 powers of two within one tile) or makes it
  //    non-finite marks the workgroup, which then recomputes its rows with
  //    EXACT.
  constexpr int PSPAN = 92;
  constexpr int MAX0 = 66, MAXN = 56;
  constexpr int DEC = MAX0 + MAXN;  // slots DEC .. DEC+3: the rescale test of each query block
  // The eight tile loads of a wavefront (K(t+2), then V(t+1)) go out one every
  // four slots from DMA0 on.
  constexpr int DMA0 = 2;
  auto tile_slots = [&](auto exact_c, bool maskn, int t, f32x4* sc, f32x4* sn, const bf16* kn, const bf16* vs,
                        bf16* kdma, bf16* vdma, bool& bad) {
    constexpr bool EXACT = decltype(exact_c)::value;
    const uint32_t kt_base = t + 2 < ntiles ? tile_base(t + 2) : 0xF0000000u;
    const uint32_t vt_base = t + 1 < ntiles ? tile_base(t + 1) : 0xF0000000u;
    const auto rk2 = tile_rsrc(min(t + 2, ntiles - 1), 0);
    const auto rv1 = tile_rsrc(min(t + 1, ntiles - 1), 1);
    // operand n: K block n / 4, k-step n % 4 (n < 16); Vᵀ key chunk (n-16) / 8, block (n-16) % 8
    auto oread = [&](int n) {
      if (n < 16) return *reinterpret_cast<const bf16x8*>(kn + koff(n / 4, n % 4));
      const int c = (n - 16) / DB, db = (n - 16) % DB;
      const bf16x4 lo = lds_read_tr4(vs + voff(db, c, 0));
      const bf16x4 hi = lds_read_tr4(vs + voff(db, c, 1));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    bf16x8 op[LOOK + 1];
    u32x4 pw[QB][2];  // Pᵀ(t) of query block j, key chunk c, as packed bf16 pairs
    float px[32][2];  // score pair pi: s·scale·log2e − m, then its exp
    float pt[32];     // and the pair's sum
    float mx[QB];
#pragma unroll
    for (int j = 0; j < QB; ++j) mx[j] = kNegInf;
    uint64_t need[QB];
    static_for<0, LOOK>([&](auto ic) __attribute__((always_inline)) { op[ic.value] = oread(ic.value); });
    static_for<0, NSL>([&](auto sc_) __attribute__((always_inline)) {
      constexpr int s = decltype(sc_)::value;
      constexpr int n = s / 4, j = s % 4;
      if constexpr (j == 0 && n + LOOK < 32) op[(n + LOOK) % (LOOK + 1)] = oread(n + LOOK);
      if constexpr (n < 16) {
        constexpr int kb = n / 4, kk = n % 4;
        if constexpr (kk == 0)
          mfma16_s0_here(sn[4 * kb + j], op[n % (LOOK + 1)], qreg[j][kk]);
        else
          mfma16_s_here(sn[4 * kb + j], op[n % (LOOK + 1)], qreg[j][kk]);
      } else {
        constexpr int c = (n - 16) / DB, db = (n - 16) % DB;
        mfma16_o_here(oacc[db][j], op[n % (LOOK + 1)], __builtin_bit_cast(bf16x8, pw[j][c]));
      }
      // score pairs: pi = 16c + 4jp + 2h + w (key chunk c, query block jp, key block 2c + h, registers 2w, 2w+1)
      // Softmax work of this slot, at most one operation of each kind (the
      // fma slots of the 64 values are distinct): the fma of value xf, the
      // exp of value xe (its fma was in the previous slot), the pack and pair
      // sum of the pair whose second fma was two slots back, and the row sum
      // of the pair one slot older.  These are plain operations, not asm
      // statements: the compiler sees what they are and pads only the waits
      // the hardware needs.  As asm statements they cost a wait state before
      // nearly every one of them (the compiler counts an asm statement as no
      // wait at all and treats its result as possibly that of a
      // transcendental).  The compiler keeps the fma, exp and sums within a
      // slot or two of where they are written here and issues the packs in
      // groups of four, well ahead of their products (measured slightly
      // faster than packs pinned one per slot).
      constexpr int xf = value_at_slot<PSPAN>(s), xe = value_at_slot<PSPAN>(s - 1);
      constexpr int xp = value_at_slot<PSPAN>(s - 2), xa = value_at_slot<PSPAN>(s - 3);
      // value x: pair pi = x / 2 = 16c + 4jp + 2h + w (key chunk c, query block
      // jp, key block 2c + h, registers 2w, 2w+1), register x % 2 of the pair
      auto score = [&](auto xc) -> float {
        constexpr int x = decltype(xc)::value, pi = x / 2;
        constexpr int c = pi / 16, jp = (pi / 4) % 4, h = (pi / 2) % 2, w = pi % 2;
        return sc[4 * (2 * c + h) + jp][2 * w + x % 2];
      };
      if constexpr (xf >= 0)
        px[xf / 2][xf % 2] = __builtin_fmaf(score(std::integral_constant<int, xf>{}), scale_log2, -m_run[(xf / 8) % 4]);
      if constexpr (xe >= 0) px[xe / 2][xe % 2] = exp2_fast(px[xe / 2][xe % 2]);
      if constexpr (xp >= 0 && xp % 2 == 1) {
        constexpr int pi = xp / 2, c = pi / 16, jp = (pi / 4) % 4, h = (pi / 2) % 2, w = pi % 2;
        static_assert(s <= 64 + 32 * c + jp - 2, "a Pᵀ operand must be packed two slots before its product");
        static_assert(s + 1 < DEC, "the row sums are complete before their test");
        pw[jp][c][2 * h + w] = pack_bf16x2(px[pi][0], px[pi][1]);
        pt[pi] = px[pi][0] + px[pi][1];
      }
      if constexpr (xa >= 0 && xa % 2 == 1) l_run[(xa / 8) % 4] += pt[xa / 2];  // fp32 sum of the unrounded p
      if constexpr (EXACT) {
        // max of S(t+1): value pair v of block (kb, jq) = (v / 8, (v / 2) % 4), registers 2(v % 2)..
        static_for<0, 32>([&](auto vc_) __attribute__((always_inline)) {
          constexpr int v = decltype(vc_)::value;
          constexpr int kb = v / 8, jq = (v / 2) % 4, r = 2 * (v % 2);
          constexpr int at = MAX0 + (v * MAXN) / 32;
          static_assert(at >= 16 * kb + 12 + jq + 4, "a max reads its block four products after the block's last");
          static_assert(at < DEC, "the max of S(t+1) precedes its test");
          if constexpr (at == s) max3_here(mx[jq], sn[4 * kb + jq][r], sn[4 * kb + jq][r + 1]);
        });
        // lazy-rescale test of query block s - DEC: any lane whose part of the
        // row max exceeds the reference by the threshold
        if constexpr (s >= DEC && s < DEC + QB)
          need[s - DEC] = __builtin_amdgcn_ballot_w64(mx[s - DEC] * scale_log2 > m_run[s - DEC] + kRescaleThreshold);
      } else {
        // sum test of query block s - DEC: any lane whose part of the row sum
        // exceeds kSumRescale or is not a number
        if constexpr (s >= DEC && s < DEC + QB)
          need[s - DEC] = __builtin_amdgcn_ballot_w64(!(l_run[s - DEC] <= kSumRescale));
      }
      if constexpr (s >= DMA0 && (s - DMA0) % 4 == 0 && (s - DMA0) / 4 < 2 * DMA_PER_WAVE) {
        constexpr int i = (s - DMA0) / 4;
        if constexpr (i < DMA_PER_WAVE)
          issue_k1(kdma, rk2, kt_base, i);
        else
          issue_v1(vdma, rv1, vt_base, i - DMA_PER_WAVE);
      }
      __builtin_amdgcn_sched_barrier(0);
    });

    if constexpr (EXACT) {
      if (t + 1 < wnt) {
        if (maskn) {
          mask((t + 1) * kBC, sn);
#pragma unroll
          for (int j = 0; j < QB; ++j) {
            mx[j] = kNegInf;
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
              for (int r = 0; r < 4; ++r) mx[j] = fmaxf(mx[j], sn[4 * kb + j][r]);
            need[j] = __builtin_amdgcn_ballot_w64(mx[j] * scale_log2 > m_run[j] + kRescaleThreshold);
          }
        }
#pragma unroll
        for (int j = 0; j < QB; ++j) {
          if (need[j]) {
            mfma_drain();
            const float mt = quad_max(mx[j]) * scale_log2;
            const float m_new = fmaxf(m_run[j], mt);
            const float alpha = exp2_fast(m_run[j] - m_new);
            l_run[j] *= alpha;
            scale_out(j, alpha);
            m_run[j] = m_new;
          }
        }
      }
    } else {
      if (t + 1 < wnt && maskn) mask((t + 1) * kBC, sn);
      // Every tile, the last one included (a sum past kSumLimit there still
      // means a partial output may have overflowed).
#pragma unroll
      for (int j = 0; j < QB; ++j) {
        if (need[j]) {
          mfma_drain();
          const float lq = quad_sum(l_run[j]);  // the row sum of this lane's query
          const bool over = !(lq < kSumLimit);
          bad = bad || over;
          // lq = f·2^e with f in [0.5, 1): scale by 2^-e (exact) where lq > kSumRescale
          const int e = (!over && lq > kSumRescale) ? __builtin_amdgcn_frexp_expf(lq) : 0;
          const float alpha = __builtin_amdgcn_ldexpf(1.f, -e);
          l_run[j] *= alpha;
          scale_out(j, alpha);
          m_run[j] += (float)e;
        }
      }
    }
  };

  // The whole key loop of this workgroup; EXACT as above.  Returns (the same
  // in every wave) whether the sum check found a row it cannot bound.
  auto run = [&](auto exact_c) {
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int j = 0; j < QB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) oacc[b][j][r] = 0.f;
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      m_run[j] = kNegInf;
      l_run[j] = 0.f;
    }
    if (ntiles > 0) issue_k(kbuf0, 0);
    if (ntiles > 1) issue_k(kbuf1, 1);
    if (ntiles > 0) issue_v(vbuf0, 0);
    wait_vm_all();
    __syncthreads();
    f32x4 sa[KB * QB], sb[KB * QB];
    if (wnt > 0) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int kk = 0; kk < KC; ++kk) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(kbuf0 + koff(kb, kk));
#pragma unroll
          for (int j = 0; j < QB; ++j) {
            if (kk == 0)
              mfma16_s0(sa[4 * kb + j], a, qreg[j][kk]);
            else
              mfma16_s(sa[4 * kb + j], a, qreg[j][kk]);
          }
        }
      mfma_drain();
      mask(0, sa);
#pragma unroll
      for (int j = 0; j < QB; ++j) {
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sa[4 * kb + j][r]);
        // a query with no visible key keeps a finite reference (its p are all 0)
        const float m0 = quad_max(mx);
        m_run[j] = m0 == kNegInf ? 0.f : m0 * scale_log2;
      }
    }

    bool bad = false;
    auto step = [&](int t, f32x4* sc, f32x4* sn, bf16* kc, bf16* kn, bf16* vc, bf16* vn) {
      const int k0 = t * kBC;
      wait_vm_all();
      __syncthreads();  // K(t+1) and V(t) resident for every wave; tile t-1 fully consumed
      if (k0 + kBC > Nk) {  // tail tile: V rows past the last key must read as zero
        const int first = Nk - k0;
        for (int idx = tid; idx < (kBC - first) * CPR; idx += THREADS) {
          const u32x4 z = {0u, 0u, 0u, 0u};
          *reinterpret_cast<u32x4*>(vc + (first + idx / CPR) * D + (idx % CPR) * 8) = z;
        }
        __syncthreads();
      }
      if (t >= wnt) {  // nothing to compute here, but this wave's share of the loads still goes out
        if (t + 2 < ntiles) issue_k(kc, t + 2);
        if (t + 1 < ntiles) issue_v(vn, t + 1);
        return;
      }
      const int k0n = k0 + kBC;
      tile_slots(exact_c, (CAUSAL && k0n + kBC - 1 > qw + off) || (k0n + kBC > Nk), t, sc, sn, kn, vc, kc, vn, bad);
    };

    for (int t = 0; t < ntiles; t += 2) {  // unrolled by two so S(t) and S(t+1) swap registers
      step(t, sa, sb, kbuf0, kbuf1, vbuf0, vbuf1);
      if (t + 1 < ntiles) step(t + 1, sb, sa, kbuf1, kbuf0, vbuf1, vbuf0);
    }
    mfma_drain();
    // also the barrier after which the ring may be loaded again
    return __syncthreads_or(bad ? 1 : 0) != 0;
  };

  if (run(std::false_type{})) run(std::true_type{});

#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const float l_tot = quad_sum(l_run[j]);
    const int qrow = qw + 16 * j + i16;
    if (qrow >= N) continue;
    const float inv = hv.cut ? kNaN : (l_tot > 0.f ? 1.f / l_tot : 0.f);
    bf16* Orow = O + hv.q_off + (size_t)qrow * hv.qs;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      u32x2 w;
      w[0] = pack_bf16x2(oacc[b][j][0] * inv, oacc[b][j][1] * inv);
      w[1] = pack_bf16x2(oacc[b][j][2] * inv, oacc[b][j][3] * inv);
      *reinterpret_cast<u32x2*>(Orow + 16 * b + 4 * G) = w;
    }
    if (LSE != nullptr && G == 0)
      LSE[hv.st_off + qrow] = hv.cut ? kNaN : (l_tot > 0.f ? (m_run[j] + log2_fast(l_tot)) * kLn2 : kNegInf);
  }
}

// fp32 path: one thread per query row, keys staged through LDS 32 at a time,
// fp32 fused multiply-adds and an online softmax updated key by key.
template <int D>
__global__ __launch_bounds__(64) void fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                     const float* __restrict__ V, float* __restrict__ O,
                                                     float* __restrict__ LSE, AttnShape shape, float scale,
                                                     int causal) {
  constexpr int TK = 32;
  __shared__ float sk[TK][D];
  __shared__ float sv[TK][D];
  const int tid = threadIdx.x;
  const int row = blockIdx.x * 64 + tid;
  const int bh = blockIdx.y;
  const HeadView hv = head_view(shape, bh / shape.H, bh % shape.H, D);
  const int N = hv.L;
  if ((int)blockIdx.x * 64 >= N) return;
  float q[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = row < N ? Q[hv.q_off + (size_t)row * hv.qs + d] : 0.f;
    acc[d] = 0.f;
  }
  float m = kNegInf, l = 0.f;
  const int kend = causal ? min(N, (int)blockIdx.x * 64 + 64) : N;
  for (int k0 = 0; k0 < kend; k0 += TK) {
    __syncthreads();
    for (int i = tid; i < TK * D; i += 64) {
      const int r = i / D, d = i % D;
      const bool ok = k0 + r < N;
      sk[r][d] = ok ? K[hv.kv_off + (size_t)(k0 + r) * hv.kvs + d] : 0.f;
      sv[r][d] = ok ? V[hv.kv_off + (size_t)(k0 + r) * hv.kvs + d] : 0.f;
    }
    __syncthreads();
    for (int j = 0; j < TK; ++j) {
      const int key = k0 + j;
      if (key >= N || (causal && key > row)) continue;
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = __builtin_fmaf(q[d], sk[j][d], s);
      s *= scale;
      if (s > m) {
        const float a = expf(m - s);
        l *= a;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] *= a;
        m = s;
      }
      const float p = expf(s - m);
      l += p;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(p, sv[j][d], acc[d]);
    }
  }
  if (row >= N) return;
  const float inv = hv.cut ? kNaN : 1.f / l;
#pragma unroll
  for (int d = 0; d < D; ++d) O[hv.q_off + (size_t)row * hv.qs + d] = acc[d] * inv;
  if (LSE != nullptr) LSE[hv.st_off + row] = hv.cut ? kNaN : m + logf(l);
}

template <int D, bool PAGED, bool ROPE>
hipError_t launch_bf16(const ForwardArgs& a) {
  const int nqb = (a.s.N + kBR - 1) / kBR;
  const dim3 grid((unsigned)(nqb * a.s.B * a.s.H)), block(kThreads);
  const float sl2 = a.scale * kLog2e;
  auto* q = static_cast<const bf16*>(a.q);
  auto* k = static_cast<const bf16*>(PAGED ? a.kv.pool : a.k);
  auto* v = static_cast<const bf16*>(PAGED ? a.kv.pool : a.v);
  auto* o = static_cast<bf16*>(a.o);
  if (a.causal)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, true, PAGED, ROPE>), grid, block, 0, a.stream, q, k, v, o, a.lse, a.s,
                       a.kv, a.rope, sl2);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, false, PAGED, ROPE>), grid, block, 0, a.stream, q, k, v, o, a.lse, a.s,
                       a.kv, a.rope, sl2);
  return hipGetLastError();
}

template <bool PAGED>
hipError_t launch_w64(const ForwardArgs& a) {
  const int nqb = (a.s.N + kBR - 1) / kBR;
  const dim3 grid((unsigned)(nqb * a.s.B * a.s.H)), block(256);
  const float sl2 = a.scale * kLog2e;
  auto* q = static_cast<const bf16*>(a.q);
  auto* k = static_cast<const bf16*>(PAGED ? a.kv.pool : a.k);
  auto* v = static_cast<const bf16*>(PAGED ? a.kv.pool : a.v);
  auto* o = static_cast<bf16*>(a.o);
  if (a.causal)
    hipLaunchKernelGGL((fwd_w64_kernel<true, PAGED>), grid, block, 0, a.stream, q, k, v, o, a.lse, a.s, a.kv, sl2);
  else
    hipLaunchKernelGGL((fwd_w64_kernel<false, PAGED>), grid, block, 0, a.stream, q, k, v, o, a.lse, a.s, a.kv, sl2);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bf16_any(const ForwardArgs& a) {
  const bool paged = a.kv.pool != nullptr, rope = a.rope.cos != nullptr;
  if (D == 128 && !rope) return paged ? launch_w64<true>(a) : launch_w64<false>(a);
  if (paged) return rope ? launch_bf16<D, true, true>(a) : launch_bf16<D, true, false>(a);
  return rope ? launch_bf16<D, false, true>(a) : launch_bf16<D, false, false>(a);
}

template <int D>
hipError_t launch_f32(const ForwardArgs& a) {
  const dim3 grid((a.s.N + 63) / 64, a.s.B * a.s.H), block(64);
  hipLaunchKernelGGL((fwd_f32_kernel<D>), grid, block, 0, a.stream, static_cast<const float*>(a.q),
                     static_cast<const float*>(a.k), static_cast<const float*>(a.v), static_cast<float*>(a.o),
                     a.lse, a.s, a.scale, a.causal);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward(const ForwardArgs& a) {
  if (a.bf16) return a.d == 128 ? launch_bf16_any<128>(a) : launch_bf16_any<64>(a);
  return a.d == 128 ? launch_f32<128>(a) : launch_f32<64>(a);
}

}  // namespace fa
