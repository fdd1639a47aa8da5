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

// Rescale the output only when the running max grows by more than this many
// powers of two.  Between rescales p = 2^(s·scale·log2e − m) <= 2^8: the
// output, its normaliser and the logsumexp all use the same reference m, so
// the result is the same exact quantity (only rounding differs).
constexpr float kRescaleThreshold = 8.0f;

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

// Rotation of one feature pair (a, b) by (c, s), rounded to bf16: the exact
// rotation (a·c − b·s, a·s + b·c) rounded to nearest.  Computed in fp32, whose
// error is below e = 2^-21·(|a|+|b|)·(|c|+|s|); when the bf16 roundings of
// r − e and r + e agree, every value in between (the exact one included)
// rounds the same way.  Otherwise (rare: r within e of a rounding boundary)
// the lane recomputes the pair in fp64, where the products of bf16 and fp32
// values are exact and only the sum is rounded, and rounds that directly.
__device__ __forceinline__ void rotate_pair(float a, float b, float c, float s, uint32_t& ox, uint32_t& oy) {
  const float xr = __builtin_fmaf(a, c, -(b * s));
  const float yr = __builtin_fmaf(a, s, b * c);
  const float e = (__builtin_fabsf(a) + __builtin_fabsf(b)) * (__builtin_fabsf(c) + __builtin_fabsf(s)) * 0x1p-21f;
  const uint32_t wx = pack_bf16x2(xr - e, xr + e), wy = pack_bf16x2(yr - e, yr + e);
  ox = pack_bf16x2(xr, xr) & 0xffffu;
  oy = pack_bf16x2(yr, yr) & 0xffffu;
  if (((wx ^ (wx >> 16)) | (wy ^ (wy >> 16))) & 0xffffu) {
    const double ad = a, bd = b, cd = c, sd = s;
    ox = bf16_rne_f64(ad * cd - bd * sd);
    oy = bf16_rne_f64(ad * sd + bd * cd);
  }
}

// Rotate the feature pairs (x[j], y[j]) of 8 bf16 values each by the angles
// whose cosines / sines are c[j], s[j] (rotate_pair per pair).
__device__ __forceinline__ void rotate8(bf16x8& x, bf16x8& y, const float* c, const float* s) {
  u32x4 wx, wy;
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    uint32_t x0, y0, x1, y1;
    rotate_pair((float)x[j], (float)y[j], c[j], s[j], x0, y0);
    rotate_pair((float)x[j + 1], (float)y[j + 1], c[j + 1], s[j + 1], x1, y1);
    wx[j / 2] = x0 | (x1 << 16);
    wy[j / 2] = y0 | (y1 << 16);
  }
  x = __builtin_bit_cast(bf16x8, wx);
  y = __builtin_bit_cast(bf16x8, wy);
}
// Same for the interleaved pairing: pairs (x[2j], x[2j+1]), angles c[j], s[j].
__device__ __forceinline__ void rotate8_interleaved(bf16x8& x, const float* c, const float* s) {
  u32x4 w;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t r0, r1;
    rotate_pair((float)x[2 * j], (float)x[2 * j + 1], c[j], s[j], r0, r1);
    w[j] = r0 | (r1 << 16);
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
  // place in LDS: once per workgroup and tile, every thread one item.
  auto rope_k = [&](bf16* ks, int k0) {
    if constexpr (ROPE && !PAGED) {
      if (!rope.interleaved) {
        constexpr int PAIRS = CPR / 2;  // chunk c pairs with chunk c + CPR/2
        for (int w = tid; w < kTileRows * PAIRS; w += kThreads) {
          const int r = w / PAIRS, c = w % PAIRS;
          const int pos = min(k0 + r, rope.rows - 1);
          bf16x8* px = reinterpret_cast<bf16x8*>(ks + r * D + ((c ^ rm_swz<D>(r)) << 3));
          bf16x8* py = reinterpret_cast<bf16x8*>(ks + r * D + (((c + PAIRS) ^ rm_swz<D>(r)) << 3));
          float cs[8], sn[8];
          load_f32<8>(cs, rope.cos + (size_t)pos * (D / 2) + 8 * c);
          load_f32<8>(sn, rope.sin + (size_t)pos * (D / 2) + 8 * c);
          bf16x8 x = *px, y = *py;
          rotate8(x, y, cs, sn);
          *px = x;
          *py = y;
        }
      } else {
        for (int w = tid; w < kTileRows * CPR; w += kThreads) {
          const int r = w / CPR, c = w % CPR;
          const int pos = min(k0 + r, rope.rows - 1);
          bf16x8* px = reinterpret_cast<bf16x8*>(ks + r * D + ((c ^ rm_swz<D>(r)) << 3));
          float cs[4], sn[4];
          load_f32<4>(cs, rope.cos + (size_t)pos * (D / 2) + 4 * c);
          load_f32<4>(sn, rope.sin + (size_t)pos * (D / 2) + 4 * c);
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
  if (ntiles > 1) issue_k(kbuf1, 1);
  if (ntiles > 0) issue_v(vbuf0, 0);
  wait_vm_all();
  __syncthreads();
  if (ntiles > 0) rope_k(kbuf0, 0);
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
  auto step = [&](int t, f32x16* sc, f32x16* sn, bf16* kc, bf16* kn, bf16* vc, bf16* vn) {
    const int k0 = t * kBC;
    wait_vm_all();
    __syncthreads();  // K(t+1) and V(t) resident for every wave; tile t-1 fully consumed
    if (t + 2 < ntiles) issue_k(kc, t + 2);
    if (t + 1 < ntiles) issue_v(vn, t + 1);
    if (k0 + kBC > Nk) {  // tail tile: V rows past the last key must read as zero, whatever the loads left
      const int first = Nk - k0;
      for (int idx = tid; idx < (kBC - first) * CPR; idx += kThreads) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(vc + (first + idx / CPR) * D + (idx % CPR) * 8) = z;
      }
      __syncthreads();
    }
    if (t + 1 < ntiles) rope_k(kn, (t + 1) * kBC);
    if (t >= wnt) return;
    const int k0n = k0 + kBC;
    tile_slots((CAUSAL && k0n + kBC - 1 > qw + off) || (k0n + kBC > Nk), t, sc, sn, kn, vc);
  };

  for (int t = 0; t < ntiles; t += 2) {  // unrolled by two so S(t) and S(t+1) swap registers
    step(t, sa, sb, kbuf0, kbuf1, vbuf0, vbuf1);
    if (t + 1 < ntiles) step(t + 1, sb, sa, kbuf1, kbuf0, vbuf1, vbuf0);
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
// per SIMD.  Each K and Vᵀ operand read from
// LDS feeds two products (query blocks j = 0, 1), halving LDS traffic per
// FLOP; the output accumulators live in accumulation registers.
template <bool CAUSAL, bool PAGED>
__global__ __launch_bounds__(256, 1) void fwd_w64_kernel(const bf16* __restrict__ Q, const bf16* __restrict__ K,
                                                         const bf16* __restrict__ V, bf16* __restrict__ O,
                                                         float* __restrict__ LSE, AttnShape shape, PagedKV pkv,
                                                         float scale_log2) {
  constexpr int D = 128;
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int TILE = kTileRows * D;
  constexpr int CPR = D / 8;
  constexpr int WAVES = 4;
  constexpr int THREADS = 64 * WAVES;
  constexpr int ROWS_PER_DMA = 64 / CPR;
  constexpr int DMA_PER_WAVE = kTileRows / ROWS_PER_DMA / WAVES;
  __shared__ __attribute__((aligned(1024))) bf16 kbuf0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 kbuf1[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 vbuf0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 vbuf1[TILE];
  __shared__ int ptab[PAGED ? kMaxPrefillPages : 1];  // this sequence's pool pages

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, n = lane & 31;
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
  const int qw = q0 + wave * 64;  // this wave's first query; query block j holds qw + 32j ..

  // Qᵀ as the B operand of both query blocks (zeros past N).
  bf16x8 qreg[2][KSTEPS];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
      qreg[j][kk] = __builtin_bit_cast(
          bf16x8, buf_load16(rq, (uint32_t)(qw + 32 * j + n) * (hv.qs * 2) + (16 * kk + 8 * g) * 2));

  // Direct-to-LDS loads: rows (wave·DMA_PER_WAVE + i)·ROWS_PER_DMA + lane / CPR
  // of a tile; the swizzled chunk offsets are recomputed at each issue.
  const int dma_row = lane / CPR, dma_pc = lane % CPR;
  auto dma_off = [&](int i, bool vtile) {
    const int row = (wave * DMA_PER_WAVE + i) * ROWS_PER_DMA + dma_row;
    return (uint32_t)row * (kvs * 2) + ((dma_pc ^ (vtile ? v_swz<D>(row) : rm_swz<D>(row))) << 4);
  };
  // Spread issue (one load at a time inside the slots): row r = 16·wave + 4i + dma_row,
  // so the V chunk swizzle (a function of r % 4) is the same for every i and
  // the K one is (dma_pc ^ dma_row) ^ (8(i & 1) + 4(i >> 1)); the row offset's
  // i- and tile-dependent part is uniform.  `tbase` is the tile's byte offset,
  // or an offset past every buffer for a load that is not needed (it then
  // reads nothing and writes only a slot no one reads again).
  const uint32_t drow = (uint32_t)(16 * wave + dma_row) * (uint32_t)(kvs * 2);
  const uint32_t kch = (uint32_t)(dma_pc ^ dma_row) << 4;
  const uint32_t vlane = drow + ((uint32_t)(dma_pc ^ v_swz<D>(dma_row)) << 4);
  auto issue_k1 = [&](bf16* slot, __amdgpu_buffer_rsrc_t r, uint32_t tbase, int i) {
    const uint32_t ch = kch ^ ((uint32_t)(8 * (i & 1) + 4 * (i >> 1)) << 4);
    lds_dma16(r, slot + (wave * DMA_PER_WAVE + i) * 512, drow + ch + (tbase + (uint32_t)(4 * i * kvs * 2)));
  };
  auto issue_v1 = [&](bf16* slot, __amdgpu_buffer_rsrc_t r, uint32_t tbase, int i) {
    lds_dma16(r, slot + (wave * DMA_PER_WAVE + i) * 512, vlane + (tbase + (uint32_t)(4 * i * kvs * 2)));
  };
  auto issue_k = [&](bf16* slot, int t) {
    const auto r = tile_rsrc(t, 0);
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i)
      lds_dma16(r, slot + (wave * DMA_PER_WAVE + i) * 512, dma_off(i, false) + tile_base(t));
  };
  auto issue_v = [&](bf16* slot, int t) {
    const auto r = tile_rsrc(t, 1);
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i)
      lds_dma16(r, slot + (wave * DMA_PER_WAVE + i) * 512, dma_off(i, true) + tile_base(t));
  };

  // LDS operand offsets (elements).  K: rows perm_row(n), 16-byte chunk
  // (2kk + g) ^ (n % 16) = 2(kk ^ c1) + (g ^ c0) with c = n % 16: one base and
  // an XOR per k-step.  Vᵀ: chunk (4b + x) ^ v_swz(row) with x < 4 is
  // 4(b ^ s2) + (x ^ (v_swz & 3)), s2 = v_swz >> 2: one base and an XOR per d block.
  const int kc = n & (CPR - 1);
  const int kbase = perm_row(n) * D + ((g ^ (kc & 1)) << 3);
  const int kx = (kc >> 1) << 4;
  auto koff = [&](int kk) { return kbase + ((kk << 4) ^ kx); };
  const int G = lane >> 4, j16 = lane & 15;
  const int vrow = 8 * (G >> 1) + (j16 >> 2);
  const int vsw = v_swz<D>(vrow);
  const int vx = 2 * (G & 1) + ((4 * (j16 & 3)) >> 3);
  const int vbase = vrow * D + ((vx ^ (vsw & 3)) << 3) + ((4 * (j16 & 3)) & 7);
  const int vs2 = (vsw >> 2) << 5;
  auto voff = [&](int b) { return vbase + ((b << 5) ^ vs2); };

  // s[2 kb + j]: Sᵀ block of keys 32kb.., queries 32j.. (register r: key crow(kb, r, g), query n).
  auto mask = [&](int k0, f32x16* s) {
    if ((CAUSAL && k0 + kBC - 1 > qw + off) || (k0 + kBC > Nk)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + crow(kb, r, g);
            const bool dead = (key >= Nk) || (CAUSAL && key > qw + 32 * j + n + off);
            s[2 * kb + j][r] = dead ? kNegInf : s[2 * kb + j][r];
          }
    }
  };

  f32x16 oacc[DBLK][2];
#pragma unroll
  for (int b = 0; b < DBLK; ++b)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[b][j][r] = 0.f;
  float m_run[2] = {kNegInf, kNegInf};
  float l_run[2] = {0.f, 0.f};

  const int kv_end = CAUSAL ? max(min(Nk, q0 + kBR + off), 0) : Nk;
  const int ntiles = (kv_end + kBC - 1) / kBC;
  const int wlast = min(qw + 63, N - 1) + off;  // the wave's last visible key (causal)
  const int wnt = (qw >= N) ? 0 : (CAUSAL ? (wlast < 0 ? 0 : min(ntiles, wlast / kBC + 1)) : ntiles);

  if (ntiles > 0) issue_k(kbuf0, 0);
  if (ntiles > 1) issue_k(kbuf1, 1);
  if (ntiles > 0) issue_v(vbuf0, 0);
  wait_vm_all();
  __syncthreads();
  f32x16 sa[4], sb[4];
  if (wnt > 0) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kbuf0 + kb * 32 * D + koff(kk));
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (kk == 0)
            mfma_s0(sa[2 * kb + j], a, qreg[j][kk]);
          else
            mfma_s(sa[2 * kb + j], a, qreg[j][kk]);
        }
      }
    mfma_drain();
    mask(0, sa);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sa[2 * kb + j][r]);
      m_run[j] = xhalf_max(mx) * scale_log2;
    }
  }

  // One tile: NS slots of S(t+1) (one K read, two products each), then NP
  // slots of Oᵀ += Vᵀ·Pᵀ (one Vᵀ read, two products each); P(t) pairs and
  // the max of S(t+1) ride along as in the 32-query kernel.
  constexpr int LOOK = kLook;
  constexpr int NS = 2 * KSTEPS;
  constexpr int NP = 4 * DBLK;
  constexpr int NT = NS + NP;
  // Softmax of S(t): value x's fma in half-slot fma_slot<PSPAN>(x) (the last
  // pack lands two half-slots before the product that reads it).  Max of
  // S(t+1): key block 0's values over half-slots MAXA .. MAXB-1, key block 1's
  // over MAXB .. MAXN-1, each block at least five half-slots after its last
  // product.
  constexpr int PSPAN = 54;
  constexpr int MAXA = 20, MAXB = 36, MAXN = 56;
  constexpr int DEC = 2 * NT - 6;    // half-slots DEC, DEC + 1: its reduction and rescale test
  // The loads of K(t+2) and V(t+1) go out one instruction every other
  // half-slot from DMA0 on: issued in one burst, the four wavefronts' loads
  // queue behind each other in the CU's memory pipeline and stall the issue.
  constexpr int DMA0 = 1;
  auto tile_slots = [&](bool maskn, int t, f32x16* sc, f32x16* sn, const bf16* kn, const bf16* vs,
                        bf16* kdma, bf16* vdma) {
    const uint32_t kt_base = t + 2 < ntiles ? tile_base(t + 2) : 0xF0000000u;
    const uint32_t vt_base = t + 1 < ntiles ? tile_base(t + 1) : 0xF0000000u;
    const auto rk2 = tile_rsrc(min(t + 2, ntiles - 1), 0);
    const auto rv1 = tile_rsrc(min(t + 1, ntiles - 1), 1);
    auto kread = [&](int i) {
      return *reinterpret_cast<const bf16x8*>(kn + (i / KSTEPS) * 32 * D + koff(i % KSTEPS));
    };
    auto vread = [&](int jj) {  // Vᵀ operand: key chunk jj / DBLK, d block jj % DBLK
      const bf16* base = vs + voff(jj % DBLK) + 16 * (jj / DBLK) * D;
      const bf16x4 lo = lds_read_tr4(base);
      const bf16x4 hi = lds_read_tr4(base + 4 * D);
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    float m_use[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) m_use[j] = (m_run[j] == kNegInf) ? 0.f : m_run[j];
    bf16x8 op[LOOK + 1];
    u32x4 pw[2][4];  // P(t) of query block j, keys 16kk .. as packed bf16 pairs
    float px[32][2];  // score pair pi: s·scale·log2e − m, then its exp
    float pt[32];     // and the pair's sum
    float nm[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) nm[j] = -m_use[j];
    float mx[2] = {kNegInf, kNegInf};
    float mt[2];
    uint64_t need[2];
    // max across the lane halves, scaled, and the lazy-rescale test
    auto test = [&](int j) __attribute__((always_inline)) {
      mt[j] = xhalf_max(mx[j]) * scale_log2;
      need[j] = __builtin_amdgcn_ballot_w64(mt[j] > m_run[j] + kRescaleThreshold);
    };
    static_for<0, LOOK>([&](auto ic) __attribute__((always_inline)) { op[ic.value] = kread(ic.value); });
    // Half-slots: one product each, so that with one wavefront per SIMD the
    // VALU work issues between consecutive products instead of waiting behind
    // a second one for the matrix pipe.
    static_for<0, 2 * NT>([&](auto hc) __attribute__((always_inline)) {
      constexpr int hs = decltype(hc)::value;
      constexpr int sl = hs / 2, j = hs % 2;
      constexpr int ahead = sl + LOOK;
      if constexpr (j == 0) {
        if constexpr (ahead < NS)
          op[ahead % (LOOK + 1)] = kread(ahead);
        else if constexpr (ahead < NT)
          op[ahead % (LOOK + 1)] = vread(ahead - NS);
      }
      if constexpr (sl < NS) {
        constexpr int kb = sl / KSTEPS, kk = sl % KSTEPS;
        if constexpr (kk == 0)
          mfma_s0_here(sn[2 * kb + j], op[sl % (LOOK + 1)], qreg[j][kk]);
        else
          mfma_s_here(sn[2 * kb + j], op[sl % (LOOK + 1)], qreg[j][kk]);
      } else {
        constexpr int jj = sl - NS;
        constexpr int kk = jj / DBLK, b = jj % DBLK;
        mfma_o_here(oacc[b][j], op[sl % (LOOK + 1)], __builtin_bit_cast(bf16x8, pw[j][kk]));
      }
      // score pairs: pi = 8 kk + 4 jp + w  (kk = key chunk, jp = query block, w = pair inside it)
      static_for<0, 32>([&](auto pic) __attribute__((always_inline)) {
        constexpr int pi = decltype(pic)::value;
        constexpr int kk = pi / 8, jp = (pi / 4) % 2, w = pi % 4;
        constexpr int kb = kk / 2, r = 8 * (kk % 2) + 2 * w;
        constexpr int f0 = fma_slot<PSPAN>(2 * pi), f1 = fma_slot<PSPAN>(2 * pi + 1), pk = f1 + 2;
        static_assert(pk <= 2 * NS + 8 * kk + jp - 2, "a P chunk must be packed two half-slots before its product");
        if constexpr (f0 == hs) fma_here(px[pi][0], sc[2 * kb + jp][r], scale_log2, nm[jp]);
        if constexpr (f1 == hs) fma_here(px[pi][1], sc[2 * kb + jp][r + 1], scale_log2, nm[jp]);
        if constexpr (f0 + 1 == hs) exp2_here(px[pi][0], px[pi][0]);
        if constexpr (f1 + 1 == hs) exp2_here(px[pi][1], px[pi][1]);
        if constexpr (pk == hs) {
          uint32_t packed;
          pack_here(packed, px[pi][0], px[pi][1]);
          pw[jp][kk][w] = packed;
          add_here(pt[pi], px[pi][0], px[pi][1]);
        }
        if constexpr (pk + 1 == hs) accumulate_here(l_run[jp], pt[pi]);  // fp32 sum of the unrounded p
      });
      static_for<0, 32>([&](auto vc_) __attribute__((always_inline)) {
        constexpr int v = 2 * decltype(vc_)::value;  // values v, v+1 of S(t+1)
        constexpr int blk = v / 16;                  // block 2kb + j
        constexpr int at = v < 32 ? MAXA + (v * (MAXB - MAXA)) / 32 : MAXB + ((v - 32) * (MAXN - MAXB)) / 32;
        static_assert(at < DEC, "the max of S(t+1) precedes its test");
        if constexpr (at == hs) max3_here(mx[blk % 2], sn[blk][v % 16], sn[blk][v % 16 + 1]);
      });
      if constexpr (hs == DEC || hs == DEC + 1) test(hs - DEC);
      if constexpr (hs >= DMA0 && (hs - DMA0) % 2 == 0 && (hs - DMA0) / 2 < 2 * DMA_PER_WAVE) {
        constexpr int i = (hs - DMA0) / 2;
        if constexpr (i < DMA_PER_WAVE)
          issue_k1(kdma, rk2, kt_base, i);
        else
          issue_v1(vdma, rv1, vt_base, i - DMA_PER_WAVE);
      }
      __builtin_amdgcn_sched_barrier(0);
    });

    if (t + 1 < wnt) {
      if (maskn) {
        mask((t + 1) * kBC, sn);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          mx[j] = kNegInf;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx[j] = fmaxf(mx[j], sn[2 * kb + j][r]);
          test(j);
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (need[j]) {
          mfma_drain();
          const float m_new = fmaxf(m_run[j], mt[j]);
          const float alpha = exp2_fast(m_run[j] - m_new);
          l_run[j] *= alpha;
          // in place in the accumulation registers, one element at a time
#pragma unroll
          for (int b = 0; b < DBLK; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              float x = oacc[b][j][r];
              acc_scale(x, alpha);
              oacc[b][j][r] = x;
            }
          m_run[j] = m_new;
        }
      }
    }
  };

  auto step = [&](int t, f32x16* sc, f32x16* sn, bf16* kc, bf16* kn, bf16* vc, bf16* vn) {
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
    tile_slots((CAUSAL && k0n + kBC - 1 > qw + off) || (k0n + kBC > Nk), t, sc, sn, kn, vc, kc, vn);
  };

  for (int t = 0; t < ntiles; t += 2) {
    step(t, sa, sb, kbuf0, kbuf1, vbuf0, vbuf1);
    if (t + 1 < ntiles) step(t + 1, sb, sa, kbuf1, kbuf0, vbuf1, vbuf0);
  }
  mfma_drain();

#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int qrow = qw + 32 * j + n;
    if (qrow >= N) continue;
    const float l_tot = xhalf_sum(l_run[j]);
    const float inv = hv.cut ? kNaN : (l_tot > 0.f ? 1.f / l_tot : 0.f);
    bf16* Orow = O + hv.q_off + (size_t)qrow * hv.qs;
#pragma unroll
    for (int b = 0; b < DBLK; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u32x2 w;
        w[0] = pack_bf16x2(oacc[b][j][4 * i + 0] * inv, oacc[b][j][4 * i + 1] * inv);
        w[1] = pack_bf16x2(oacc[b][j][4 * i + 2] * inv, oacc[b][j][4 * i + 3] * inv);
        *reinterpret_cast<u32x2*>(Orow + 32 * b + 8 * i + 4 * g) = w;
      }
    if (LSE != nullptr && g == 0)
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
