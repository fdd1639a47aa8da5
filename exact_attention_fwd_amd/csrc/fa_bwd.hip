// Recomputing backward of exact attention for gfx950.
//
// The forward keeps only the row logsumexp; here every probability tile is
// rebuilt on chip as P = 2^(s·scale·log2e − LSE·log2e) from Q, K and that
// statistic, and never stored ("Flash Attention 是什么" (ai.lansai.wang),
// 技术原理 › 核心工作机制, 重计算 paragraph; 关键术语解析 §5).  With
// D_i = dO_i·O_i the gradients are
//   dV = Pᵀ dO,  dP = dO Vᵀ,  dS = P ∘ (dP − D),  dK = scale·dSᵀ Q,  dQ = scale·dS K.
//
// Three kernels, all deterministic (fixed accumulation order, no atomics):
//   bwd_delta : D_i = Σ_f dO_if O_if                    (bandwidth-bound)
//   bwd_dkdv  : a workgroup owns 128 keys (32 per wavefront) and walks the
//               query tiles that see them; S and dP are held as
//               [query rows x key column per lane], so P and dS feed the dV
//               and dK products directly as B operands.
//   bwd_dq    : a workgroup owns 128 queries and walks their key tiles, with
//               Sᵀ held as [key rows x query column per lane] as in the
//               forward.
// Q/dO (dK/dV pass) and K/V (dQ pass) tiles go HBM -> LDS with direct
// buffer loads into a two-stage ring; the transposed operands (dOᵀ, Qᵀ, Kᵀ)
// are read out of the same row-major tiles with ds_read_b64_tr_b16.
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kThreads = 256;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// D_i = dO_i · O_i.  LPR = D/8 lanes share a row, 16 bytes each.
// Rows are the rows of O/dO in memory order; in the packed layout row j is
// (token j / H, head j % H) and D_i is stored [H, total] like the LSE.
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_delta_kernel(const bf16* __restrict__ O, const bf16* __restrict__ dO,
                                                             const float* __restrict__ LSE, float* __restrict__ delta,
                                                             float* __restrict__ lse2, long long rows, int H,
                                                             long long total, int packed) {
  constexpr int LPR = D / 8;
  constexpr int RPB = kThreads / LPR;  // rows per block pass
  const int c = threadIdx.x % LPR;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / LPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(O + row * D + c * 8);
    const u32x4 b = *reinterpret_cast<const u32x4*>(dO + row * D + c * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = __builtin_fmaf(__uint_as_float(a[i] << 16), __uint_as_float(b[i] << 16), acc);
      acc = __builtin_fmaf(__uint_as_float(a[i] & 0xffff0000u), __uint_as_float(b[i] & 0xffff0000u), acc);
    }
  }
  acc += dpp<0xB1>(acc);
  acc += dpp<0x4E>(acc);
  acc += dpp<0x141>(acc);
  if (LPR == 16) acc += dpp<0x140>(acc);
  if (row < rows && c == 0) {
    const long long i = packed ? (row % H) * total + row / H : row;
    delta[i] = -acc;            // −D_i: a dP accumulator can start from it
    lse2[i] = LSE[i] * kLog2e;  // the exponent base the tiles use
  }
}

// Direct-to-LDS loads of a 64-row tile of a [rows, D] matrix (row-major in
// LDS, dual-swizzled): wave w fills 1 KiB blocks w*DPW.. of the tile.
template <int D>
struct TileDma {
  static constexpr int CPR = D / 8;
  static constexpr int RPD = 64 / CPR;               // rows per 1 KiB block
  static constexpr int DPW = kTileRows / RPD / 4;    // blocks per wave
  uint32_t off[DPW];
  int base_blk;
  // `stride`: elements between consecutive rows of the source matrix.
  __device__ __forceinline__ void init(int wave, int lane, int stride) {
    base_blk = wave * DPW;
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      const int row = (base_blk + i) * RPD + lane / CPR;
      off[i] = (uint32_t)row * (uint32_t)(stride * 2) + (((lane % CPR) ^ dual_swz<D>(row)) << 4);
    }
  }
  // rows row0 .. row0+63
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t r, bf16* tile, int row0, int stride) const {
#pragma unroll
    for (int i = 0; i < DPW; ++i)
      lds_dma16(r, tile + (base_blk + i) * 512, off[i] + (uint32_t)row0 * (uint32_t)(stride * 2));
  }
};

// Per-lane element offsets of the two operand reads of a dual-swizzled tile.
// The second half of a transposed read (rows +4) sits at the same per-lane
// distance from the first for every d block, so one delta is kept.
template <int D>
struct TileReads {
  static constexpr int KSTEPS = D / 16, DBLK = D / 32;
  // row-major A operand: row perm_row(n) (+32 kb), chunk (2kk + g) ^ s with
  // s = dual_swz(row), i.e. 2(kk ^ s/2) + (g ^ s%2): a base and an XOR per k-step
  int rmb, rmx;
  int tr[DBLK];    // transposed A operand, first half: rows 8(G>>1) + j/4 (+16 kk), column 32b + 16(G&1) + 4(j%4)
  int trd;         // second half (rows +4) minus first half
  __device__ __forceinline__ void init(int lane) {
    const int g = lane >> 5, n = lane & 31;
    const int pr = perm_row(n);
    const int sw = dual_swz<D>(pr);
    rmb = pr * D + ((g ^ (sw & 1)) << 3);
    rmx = (sw >> 1) << 4;
    const int G = lane >> 4, j = lane & 15;
    auto off = [&](int b, int c) {
      const int row = 8 * (G >> 1) + 4 * c + (j >> 2);
      const int col = 32 * b + 16 * (G & 1) + 4 * (j & 3);
      return row * D + (((col >> 3) ^ dual_swz<D>(row)) << 3) + (col & 7);
    };
#pragma unroll
    for (int b = 0; b < DBLK; ++b) tr[b] = off(b, 0);
    trd = off(0, 1) - off(0, 0);
  }
  // rows 32kb.. of the tile, k-step kk over the head dim
  __device__ __forceinline__ bf16x8 row_major(const bf16* tile, int kb, int kk) const {
    return *reinterpret_cast<const bf16x8*>(tile + kb * 32 * D + rmb + ((kk << 4) ^ rmx));
  }
  // head-dim rows 32b.., k-step kk over the tile's rows (16kk .. 16kk+15)
  __device__ __forceinline__ bf16x8 transposed(const bf16* tile, int b, int kk) const {
    const bf16* p = tile + tr[b] + 16 * kk * D;
    const bf16x4 lo = lds_read_tr4(p);
    const bf16x4 hi = lds_read_tr4(p + trd);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
};

// Zero rows [first, 64) of a row-major tile (all chunks), block-wide.
template <int D>
__device__ __forceinline__ void zero_rows(bf16* tile, int first, int tid) {
  constexpr int CPR = D / 8;
  for (int idx = tid; idx < (kTileRows - first) * CPR; idx += kThreads) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(tile + (first + idx / CPR) * D + (idx % CPR) * 8) = z;
  }
}

// ---------------------------------------------------------------------------
// dK, dV: workgroup = 128 keys of one head; wavefront w owns keys kw..kw+31
// and walks the 64-query tiles that see them (Q and dO tiles in an LDS ring).
// S = Q Kᵀ and dP = dO Vᵀ are held as [32 query rows x this lane's key], so
// P and dS feed dVᵀ += dOᵀ P and dKᵀ += Qᵀ dS directly as B operands, with
// dOᵀ and Qᵀ read transposed out of the same tiles.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ delta,
    bf16* __restrict__ dK, bf16* __restrict__ dV, AttnShape shape, float scale, float scale_log2) {
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int TILE = kTileRows * D;
  __shared__ __attribute__((aligned(1024))) bf16 smem[2 * 2 * TILE];  // [stage][Q, dO]
  __shared__ __attribute__((aligned(16))) float sstat[2][2][kTileRows];  // [stage][LSE·log2e, D]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, n = lane & 31;
  int rank, b, hkv;
  map_unit(blockIdx.x, shape.B, shape.Hkv, 1, rank, b, hkv);
  const int group = shape.H / shape.Hkv;  // query heads sharing this key/value head
  const HeadView kv = head_view(shape, b, hkv * group, D);
  const int N = kv.L;
  const int k0 = rank * 128;  // causal: the first key tiles see the most queries, so they go first
  if (k0 >= N) return;        // a shorter sequence of a packed batch
  const int kw = k0 + 32 * wave;
  const int key = kw + n;  // this lane's key column
  const auto rk = make_rsrc(K + kv.kv_off, (uint32_t)N * kv.kvs * 2);
  const auto rv = make_rsrc(V + kv.kv_off, (uint32_t)N * kv.kvs * 2);

  // Kᵀ and Vᵀ as B operands: lane (g, n) holds row `key`, features 16kk+8g.. (zeros past N).
  bf16x8 kreg[KSTEPS], vreg[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    const uint32_t off = (uint32_t)key * (kv.kvs * 2) + (16 * kk + 8 * g) * 2;
    kreg[kk] = __builtin_bit_cast(bf16x8, buf_load16(rk, off));
    vreg[kk] = __builtin_bit_cast(bf16x8, buf_load16(rv, off));
  }
  f32x16 dk[DBLK], dv[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[b][r] = 0.f;
      dv[b][r] = 0.f;
    }

  const int qstart = CAUSAL ? k0 : 0;  // k0 is a multiple of the 64-query tile
  const int tph = (N - qstart + kTileRows - 1) / kTileRows;  // query tiles per query head
  const int ntiles = tph * group;  // the group's query heads one after the other
  TileDma<D> dma;
  dma.init(wave, lane, kv.qs);  // every query head of the group has the same row stride
  TileReads<D> rd;
  rd.init(lane);
  // Query-side addressing of tile i: query head hkv*group + i / tph, rows from qstart + (i % tph)*64.
  // (Offsets stepped from the first query head's view: recomputing the view would
  // re-read the packed layout's sequence offsets from memory at every tile.)
  auto qview = [&](int i) { return step_head(kv, shape, i / tph, D); };
  auto issue = [&](int i) {
    const HeadView hq = qview(i);
    bf16* st = smem + (i & 1) * 2 * TILE;
    const int r0 = qstart + (i % tph) * kTileRows;
    dma.issue(make_rsrc(Q + hq.q_off, (uint32_t)N * hq.qs * 2), st, r0, hq.qs);
    dma.issue(make_rsrc(dO + hq.q_off, (uint32_t)N * hq.qs * 2), st + TILE, r0, hq.qs);
  };
  auto load_stat = [&](int i) {  // tid < 64: LSE·log2e, 64 <= tid < 128: D
    const HeadView hq = qview(i);
    const int q = qstart + (i % tph) * kTileRows + (tid & 63);
    float x = 0.f;
    if (tid < 128 && q < N) x = (tid < 64) ? LSE[hq.st_off + q] * kLog2e : delta[hq.st_off + q];
    return x;
  };
  float stat_next = 0.f;
  issue(0);
  stat_next = load_stat(0);

  for (int i = 0; i < ntiles; ++i) {
    const int q0 = qstart + (i % tph) * kTileRows;
    const int st = i & 1;
    if (tid < 128) sstat[st][tid >> 6][tid & 63] = stat_next;
    wait_vm_all();
    __syncthreads();  // tile i resident; tile i-1 consumed by every wave
    if (i + 1 < ntiles) {
      issue(i + 1);
      stat_next = load_stat(i + 1);
    }
    bf16* qt = smem + st * 2 * TILE;
    bf16* dot = qt + TILE;
    if (q0 + kTileRows > N) {  // tail: rows past N must be zero for the transposed products
      zero_rows<D>(qt, N - q0, tid);
      zero_rows<D>(dot, N - q0, tid);
      __syncthreads();
    }
    if (kw >= N || (CAUSAL && q0 + kTileRows - 1 < kw)) continue;  // no query of the tile sees these keys
    const float* lse2 = sstat[st][0];
    const float* dlt = sstat[st][1];

    // S = Q Kᵀ and dP = dO Vᵀ for the 32 queries of block qb.
    auto sdp = [&](int qb, f32x16& sv, f32x16& dpv) {
      sv = mfma32(rd.row_major(qt, qb, 0), kreg[0], f32x16{});
      dpv = mfma32(rd.row_major(dot, qb, 0), vreg[0], f32x16{});
#pragma unroll
      for (int kk = 1; kk < KSTEPS; ++kk) {
        sv = mfma32(rd.row_major(qt, qb, kk), kreg[kk], sv);
        dpv = mfma32(rd.row_major(dot, qb, kk), vreg[kk], dpv);
      }
    };
    // P = exp(S·scale − LSE) and dS = P ∘ (dP − D), rounded to bf16 pairs of k-steps.
    auto grads = [&](auto masked, int qb, const f32x16& sv, const f32x16& dpv, bf16x8* pk, bf16x8* dsk) {
      float p[16], ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = crow(qb, r, g);
        float pr = exp2_fast(__builtin_fmaf(sv[r], scale_log2, -lse2[qi]));
        float dsr = pr * (dpv[r] + dlt[qi]);  // dlt holds −D
        if constexpr (decltype(masked)::value) {
          const int qa = q0 + qi;
          const bool dead = qa >= N || key >= N || (CAUSAL && key > qa);
          pr = dead ? 0.f : pr;
          dsr = dead ? 0.f : dsr;
        }
        p[r] = pr;
        ds[r] = dsr;
      }
      pk[0] = pack8(p);
      pk[1] = pack8(p + 8);
      dsk[0] = pack8(ds);
      dsk[1] = pack8(ds + 8);
    };
    // dVᵀ += dOᵀ P ; dKᵀ += Qᵀ dS  (k-steps 2qb, 2qb+1 over the tile's queries)
    auto accumulate = [&](int qb, const bf16x8* pk, const bf16x8* dsk) {
#pragma unroll
      for (int b = 0; b < DBLK; ++b) {
        dv[b] = mfma32(rd.transposed(dot, b, 2 * qb), pk[0], dv[b]);
        dk[b] = mfma32(rd.transposed(qt, b, 2 * qb), dsk[0], dk[b]);
        dv[b] = mfma32(rd.transposed(dot, b, 2 * qb + 1), pk[1], dv[b]);
        dk[b] = mfma32(rd.transposed(qt, b, 2 * qb + 1), dsk[1], dk[b]);
      }
    };
    // The tile's two 32-query blocks; the masked variant is taken only on
    // diagonal and tail tiles, so the common path carries no mask arithmetic.
    auto tile_body = [&](auto masked) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        // masked tiles: skip a 32-query block that precedes the keys (causal) or lies past N
        if (decltype(masked)::value && (CAUSAL ? q0 + 32 * qb + 31 < kw : q0 + 32 * qb >= N)) continue;
        f32x16 sv, dpv;
        bf16x8 pk[2], dsk[2];
        sdp(qb, sv, dpv);
        grads(masked, qb, sv, dpv, pk, dsk);
        accumulate(qb, pk, dsk);
      }
    };
    const bool need_mask = (CAUSAL && q0 < kw + 31) || (q0 + kTileRows > N) || (kw + 32 > N);
    if (need_mask)
      tile_body(std::integral_constant<bool, true>{});
    else
      tile_body(std::integral_constant<bool, false>{});
  }

  if (kw >= N || key >= N) return;
  bf16* dKrow = dK + kv.kv_off + (size_t)key * kv.kvs;
  bf16* dVrow = dV + kv.kv_off + (size_t)key * kv.kvs;
  const float ks = kv.cut ? kNaN : scale, vs = kv.cut ? kNaN : 1.f;
#pragma unroll
  for (int b = 0; b < DBLK; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x2 wk, wv;
      wk[0] = pack_bf16x2(dk[b][4 * i] * ks, dk[b][4 * i + 1] * ks);
      wk[1] = pack_bf16x2(dk[b][4 * i + 2] * ks, dk[b][4 * i + 3] * ks);
      wv[0] = pack_bf16x2(dv[b][4 * i] * vs, dv[b][4 * i + 1] * vs);
      wv[1] = pack_bf16x2(dv[b][4 * i + 2] * vs, dv[b][4 * i + 3] * vs);
      *reinterpret_cast<u32x2*>(dKrow + 32 * b + 8 * i + 4 * g) = wk;
      *reinterpret_cast<u32x2*>(dVrow + 32 * b + 8 * i + 4 * g) = wv;
    }
}

// ---------------------------------------------------------------------------
// dK, dV for d = 128 as a software pipeline: one wavefront of 32 keys per
// SIMD, four per workgroup.  Step t runs 64 half-slots, one matrix product
// each: the first 32 compute S(t+1) = Q·Kᵀ and dP(t+1) = dO·Vᵀ of the next
// 64-query tile, the last 32 accumulate dVᵀ += dOᵀ·P(t) and dKᵀ += Qᵀ·dS(t);
// meanwhile the VALU turns S(t), dP(t) into P = 2^(s·scale·log2e −
// LSE·log2e) and dS = P ∘ (dP − D).  Every LDS operand is read LOOK
// half-slots ahead of its product.  Q/dO tiles and their LSE/D rows stream
// through a four-slot LDS ring three tiles ahead (each slot its own LDS
// object, named statically, so reads never wait on loads into other
// slots); K, V and the dK, dV accumulators stay in AGPRs.  Diagonal and tail
// tiles are masked once, on S(t), dP(t), before their step.
// ---------------------------------------------------------------------------
template <bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_pipe_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE2, const float* __restrict__ delta,
    bf16* __restrict__ dK, bf16* __restrict__ dV, AttnShape shape, float scale, float scale_log2) {
  // LSE2: the rows' logsumexp times log2(e), as the delta kernel writes it
  constexpr int D = 128;
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int TILE = kTileRows * D;
  constexpr int NA = 2 * 2 * KSTEPS;  // S and dP products of a tile (two 32-query blocks)
  constexpr int NT = 2 * NA;          // plus as many dV and dK products
  constexpr int LOOK = 3;  // half-slots between an operand read and its product (2: ~1% slower)
  constexpr int VMEM_PER_TILE = 2 * TileDma<D>::DPW + 1;  // Q, dO blocks and one statistics load per wave
  __shared__ __attribute__((aligned(1024))) bf16 qs0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 qs1[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 qs2[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 qs3[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 ds0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 ds1[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 ds2[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 ds3[TILE];
  // statistics of a tile: LSE · log2(e) of its 64 query rows, then D of those rows
  __shared__ __attribute__((aligned(16))) float ss0[2 * kTileRows];
  __shared__ __attribute__((aligned(16))) float ss1[2 * kTileRows];
  __shared__ __attribute__((aligned(16))) float ss2[2 * kTileRows];
  __shared__ __attribute__((aligned(16))) float ss3[2 * kTileRows];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, n = lane & 31;
  int rank, b, hkv;
  map_unit(blockIdx.x, shape.B, shape.Hkv, 1, rank, b, hkv);
  const int group = shape.H / shape.Hkv;
  const HeadView kv = head_view(shape, b, hkv * group, D);
  const int N = kv.L;
  const int k0 = rank * 128;
  if (k0 >= N) return;
  const int kw = k0 + 32 * wave;
  const int key = kw + n;
  const auto rk = make_rsrc(K + kv.kv_off, (uint32_t)N * kv.kvs * 2);
  const auto rv = make_rsrc(V + kv.kv_off, (uint32_t)N * kv.kvs * 2);

  bf16x8 kreg[KSTEPS], vreg[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    const uint32_t off = (uint32_t)key * (kv.kvs * 2) + (16 * kk + 8 * g) * 2;
    kreg[kk] = __builtin_bit_cast(bf16x8, buf_load16(rk, off));
    vreg[kk] = __builtin_bit_cast(bf16x8, buf_load16(rv, off));
  }
  f32x16 dk[DBLK], dv[DBLK];
#pragma unroll
  for (int bb = 0; bb < DBLK; ++bb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[bb][r] = 0.f;
      dv[bb][r] = 0.f;
    }

  const int qstart = CAUSAL ? k0 : 0;
  const int tph = (N - qstart + kTileRows - 1) / kTileRows;
  const int ntiles = tph * group;
  TileDma<D> dma;
  dma.init(wave, lane, kv.qs);
  TileReads<D> rd;
  rd.init(lane);
  auto qview = [&](int i) { return step_head(kv, shape, i / tph, D); };  // as in the kernel above
  auto first_row = [&](int i) { return qstart + (int)((unsigned)i % (unsigned)tph) * kTileRows; };
  // Tile i into a ring slot: Q and dO blocks, and 32 statistics per wave
  // (wave w: rows 32(w & 1).. of LSE for w < 2, of D for w >= 2).
  auto issue = [&](int i, bf16* qslot, bf16* dslot, float* sslot) {
    const HeadView hq = qview(i);
    const int r0 = first_row(i);
    dma.issue(make_rsrc(Q + hq.q_off, (uint32_t)N * hq.qs * 2), qslot, r0, hq.qs);
    dma.issue(make_rsrc(dO + hq.q_off, (uint32_t)N * hq.qs * 2), dslot, r0, hq.qs);
    const auto rs = make_rsrc((wave < 2 ? LSE2 : delta) + hq.st_off, (uint32_t)N * 4);
    if (lane < 8) lds_dma16(rs, sslot + 32 * wave, (uint32_t)(r0 + 32 * (wave & 1) + 4 * lane) * 4);
  };
  auto a_operand = [&](const bf16* qn, const bf16* dn, int m) {  // S/dP product m: block m/16, k-step (m%16)/2
    return rd.row_major((m & 1) ? dn : qn, m / 16, (m % 16) / 2);
  };
  auto c_operand = [&](const bf16* qc, const bf16* dc, int m) {  // dV/dK product m: block m/16, d block (m%16)/4
    return rd.transposed((m & 1) ? qc : dc, (m % 16) / 4, 2 * (m / 16) + (m % 4) / 2);
  };
  auto mask_tile = [&](int i, f32x16* s) {  // S -> -inf, dP -> 0 where the key is after the query or the row past N
    const int q0 = first_row(i);
    if (!((CAUSAL && q0 < kw + 31) || (q0 + kTileRows > N))) return;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qa = q0 + crow(qb, r, g);
        const bool dead = qa >= N || (CAUSAL && key > qa);
        s[2 * qb][r] = dead ? kNegInf : s[2 * qb][r];
        s[2 * qb + 1][r] = dead ? 0.f : s[2 * qb + 1][r];
      }
  };

  // dP accumulators of query block qb start at −D of their rows (register r:
  // row 32qb + 16(r / 8) + 8g + r % 8 of the tile's statistics), so the products
  // accumulate dP − D and dS = P ∘ (dP − D) takes one multiply per score.
  auto d_init = [&](f32x16& acc, const float* st, int qb) {
#pragma unroll
    for (int run = 0; run < 2; ++run) {
      const float4 x0 = *reinterpret_cast<const float4*>(st + kTileRows + 32 * qb + 16 * run + 8 * g);
      const float4 x1 = *reinterpret_cast<const float4*>(st + kTileRows + 32 * qb + 16 * run + 8 * g + 4);
      acc[8 * run + 0] = x0.x; acc[8 * run + 1] = x0.y; acc[8 * run + 2] = x0.z; acc[8 * run + 3] = x0.w;
      acc[8 * run + 4] = x1.x; acc[8 * run + 5] = x1.y; acc[8 * run + 6] = x1.z; acc[8 * run + 7] = x1.w;
    }
  };

  if (ntiles > 0) issue(0, qs0, ds0, ss0);
  if (ntiles > 1) issue(1, qs1, ds1, ss1);
  if (ntiles > 2) issue(2, qs2, ds2, ss2);
  wait_vm_all();
  __syncthreads();
  if (first_row(0) + kTileRows > N) {
    zero_rows<D>(qs0, N - first_row(0), tid);
    zero_rows<D>(ds0, N - first_row(0), tid);
    __syncthreads();
  }
  f32x16 sa[4], sb[4];  // [2 qb + (0: S, 1: dP − D)]
  d_init(sa[1], ss0, 0);
  d_init(sa[3], ss0, 1);
  static_for<0, NA>([&](auto mc) __attribute__((always_inline)) {
    constexpr int m = decltype(mc)::value;
    const bf16x8 a = a_operand(qs0, ds0, m);
    const bf16x8& bop = (m & 1) ? vreg[(m % 16) / 2] : kreg[(m % 16) / 2];
    if constexpr ((m % 16) / 2 == 0 && (m & 1) == 0)
      mfma_s0(sa[2 * (m / 16) + (m & 1)], a, bop);
    else
      mfma_s(sa[2 * (m / 16) + (m & 1)], a, bop);
  });
  mfma_drain();

  // kc/ds/sc: ring slot of tile t; kn/dn: of tile t+1; qd/dd/sd: the slot tile t+3 loads into (tile t-1's).
  auto step = [&](int t, f32x16* sc, f32x16* sn, const bf16* qc, const bf16* dc, const float* stc, bf16* qn,
                  bf16* dn, const float* stn, bf16* qd, bf16* dd, float* sd) {
    if (t + 2 < ntiles)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(VMEM_PER_TILE) : "memory");  // tile t+1 landed; t+2 may still fly
    else
      wait_vm_all();
    __syncthreads();  // tile t+1 resident for every wave; tile t-1 consumed by every wave
    // Tile t+3's loads go out one every other half-slot (below) rather than in
    // a burst here, where the four wavefronts' bursts queue behind each other in
    // the CU's memory pipeline.  Past the last tile they aim beyond the
    // buffers and fetch nothing, so every step issues the same number of loads.
    const uint32_t bias = t + 3 < ntiles ? 0u : 0xF0000000u;
    const unsigned i3 = (unsigned)min(t + 3, ntiles - 1), j3 = i3 / (unsigned)tph;
    const HeadView hq3 = step_head(kv, shape, (int)j3, D);
    const int r03 = qstart + (int)(i3 - j3 * (unsigned)tph) * kTileRows;
    const auto rq3 = make_rsrc(Q + hq3.q_off, (uint32_t)N * hq3.qs * 2);
    const auto rd3 = make_rsrc(dO + hq3.q_off, (uint32_t)N * hq3.qs * 2);
    const auto rs3 = make_rsrc((wave < 2 ? LSE2 : delta) + hq3.st_off, (uint32_t)N * 4);
    const uint32_t roff = (uint32_t)r03 * (uint32_t)(hq3.qs * 2) + bias;
    if (t + 1 < ntiles && first_row(t + 1) + kTileRows > N) {
      zero_rows<D>(qn, N - first_row(t + 1), tid);
      zero_rows<D>(dn, N - first_row(t + 1), tid);
      __syncthreads();
    }
    mask_tile(t, sc);

    bf16x8 op[LOOK + 1];
    u32x4 pw[2][2], dw[2][2];  // P and dS of tile t as packed bf16 pairs: [query block][k-step]
    float2 lse2[16];  // statistics of each value pair (read ahead)
    d_init(sn[1], stn, 0);
    static_for<0, LOOK>([&](auto ic) __attribute__((always_inline)) { op[ic.value] = a_operand(qn, dn, ic.value); });
    // pair pi: query block pi/8, k-step (pi%8)/4, values 8h + 2w, +1 with w = pi % 4
    constexpr int PH0 = 2, PSPAN = 44;
    static_for<0, NT>([&](auto hc) __attribute__((always_inline)) {
      constexpr int hs = decltype(hc)::value;
      constexpr int ahead = hs + LOOK;
      if constexpr (ahead < NA)
        op[ahead % (LOOK + 1)] = a_operand(qn, dn, ahead);
      else if constexpr (ahead < NT)
        op[ahead % (LOOK + 1)] = c_operand(qc, dc, ahead - NA);
      if constexpr (hs % 2 == 1 && hs / 2 <= 2 * TileDma<D>::DPW) {
        constexpr int i = hs / 2;
        if constexpr (i < TileDma<D>::DPW)
          lds_dma16(rq3, qd + (dma.base_blk + i) * 512, dma.off[i] + roff);
        else if constexpr (i < 2 * TileDma<D>::DPW)
          lds_dma16(rd3, dd + (dma.base_blk + i - TileDma<D>::DPW) * 512, dma.off[i - TileDma<D>::DPW] + roff);
        else if (lane < 8)
          lds_dma16(rs3, sd + 32 * wave, (uint32_t)(r03 + 32 * (wave & 1) + 4 * lane) * 4 + bias);
      }
      if constexpr (hs == 12) d_init(sn[3], stn, 1);  // ahead of block 1's first dP product
      if constexpr (hs < NA) {
        constexpr int m = hs;
        const bf16x8& bop = (m & 1) ? vreg[(m % 16) / 2] : kreg[(m % 16) / 2];
        if constexpr ((m % 16) / 2 == 0 && (m & 1) == 0)
          mfma_s0(sn[2 * (m / 16) + (m & 1)], op[hs % (LOOK + 1)], bop);
        else
          mfma_s(sn[2 * (m / 16) + (m & 1)], op[hs % (LOOK + 1)], bop);
      } else {
        constexpr int m = hs - NA;
        constexpr int qb = m / 16, bb = (m % 16) / 4, h = (m % 4) / 2;
        if constexpr (m & 1)
          mfma_o(dk[bb], op[hs % (LOOK + 1)], __builtin_bit_cast(bf16x8, dw[qb][h]));
        else
          mfma_o(dv[bb], op[hs % (LOOK + 1)], __builtin_bit_cast(bf16x8, pw[qb][h]));
      }
      static_for<0, 16>([&](auto pc) __attribute__((always_inline)) {
        constexpr int pi = decltype(pc)::value;
        constexpr int qb = pi / 8, h = (pi % 8) / 4, w = pi % 4;
        constexpr int at = PH0 + (pi * PSPAN) / 16;
        if constexpr (at - 2 == hs) {  // statistics of the pair's two query rows
          const int row = 32 * qb + 16 * h + 8 * g + 2 * w;
          lse2[pi] = *reinterpret_cast<const float2*>(stc + row);
        }
        if constexpr (at == hs) {
          constexpr int r = 8 * h + 2 * w;
          const float p0 = exp2_fast(__builtin_fmaf(sc[2 * qb][r], scale_log2, -lse2[pi].x));
          const float p1 = exp2_fast(__builtin_fmaf(sc[2 * qb][r + 1], scale_log2, -lse2[pi].y));
          pw[qb][h][w] = pack_bf16x2(p0, p1);
          dw[qb][h][w] = pack_bf16x2(p0 * sc[2 * qb + 1][r], p1 * sc[2 * qb + 1][r + 1]);
        }
      });
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  for (int t = 0; t < ntiles; t += 4) {
    step(t, sa, sb, qs0, ds0, ss0, qs1, ds1, ss1, qs3, ds3, ss3);
    if (t + 1 < ntiles) step(t + 1, sb, sa, qs1, ds1, ss1, qs2, ds2, ss2, qs0, ds0, ss0);
    if (t + 2 < ntiles) step(t + 2, sa, sb, qs2, ds2, ss2, qs3, ds3, ss3, qs1, ds1, ss1);
    if (t + 3 < ntiles) step(t + 3, sb, sa, qs3, ds3, ss3, qs0, ds0, ss0, qs2, ds2, ss2);
  }
  mfma_drain();

  // The key index is recomputed here (a lane count the compiler cannot hoist)
  // rather than kept live across the loop.
  int lane_e;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_e));
  const int key_e = kw + (lane_e & 31);
  if (kw >= N || key_e >= N) return;
  bf16* dKrow = dK + kv.kv_off + (size_t)key_e * kv.kvs;
  bf16* dVrow = dV + kv.kv_off + (size_t)key_e * kv.kvs;
  const float ks = kv.cut ? kNaN : scale, vs = kv.cut ? kNaN : 1.f;
  // one accumulator block at a time out of the AGPRs
  static_for<0, DBLK>([&](auto bc) __attribute__((always_inline)) {
    constexpr int bb = decltype(bc)::value;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x2 wk, wv;
      wk[0] = pack_bf16x2(dk[bb][4 * i] * ks, dk[bb][4 * i + 1] * ks);
      wk[1] = pack_bf16x2(dk[bb][4 * i + 2] * ks, dk[bb][4 * i + 3] * ks);
      wv[0] = pack_bf16x2(dv[bb][4 * i] * vs, dv[bb][4 * i + 1] * vs);
      wv[1] = pack_bf16x2(dv[bb][4 * i + 2] * vs, dv[bb][4 * i + 3] * vs);
      *reinterpret_cast<u32x2*>(dKrow + 32 * bb + 8 * i + 4 * g) = wk;
      *reinterpret_cast<u32x2*>(dVrow + 32 * bb + 8 * i + 4 * g) = wv;
    }
  });
}

// ---------------------------------------------------------------------------
// dQ: workgroup = 128 queries of one head; wavefront w owns qw..qw+31 and
// walks their 64-key tiles (K and V tiles in an LDS ring).  Sᵀ and dPᵀ are
// held as [key rows x this lane's query] as in the forward; Kᵀ for
// dQᵀ += Kᵀ dSᵀ is read transposed out of the K tile.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ delta,
    bf16* __restrict__ dQ, AttnShape shape, float scale, float scale_log2) {
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int TILE = kTileRows * D;
  constexpr int BC = kTileRows;
  // two-stage ring [K tile | V tile], each stage its own LDS object named
  // statically in the twice-unrolled loop: operand reads of one stage never
  // wait on the loads still in flight into the other, and the V operand sits
  // at a fixed offset from the K operand's address
  __shared__ __attribute__((aligned(1024))) bf16 st0[2 * TILE];
  __shared__ __attribute__((aligned(1024))) bf16 st1[2 * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, n = lane & 31;
  int rank, bi, hi;
  map_unit(blockIdx.x, shape.B, shape.H, shape.H / shape.Hkv, rank, bi, hi);
  const HeadView hv = head_view(shape, bi, hi, D);
  const int N = hv.L;
  const int nqb = (N + 127) / 128;
  if (rank >= nqb) return;  // a shorter sequence of a packed batch
  const int qblk = CAUSAL ? (nqb - 1 - rank) : rank;  // causal: the last query tiles see the most keys
  const int q0 = qblk * 128;
  const int qw = q0 + 32 * wave;
  const int qrow = qw + n;
  const auto rq = make_rsrc(Q + hv.q_off, (uint32_t)N * hv.qs * 2);
  const auto rdo = make_rsrc(dO + hv.q_off, (uint32_t)N * hv.qs * 2);
  const auto rk = make_rsrc(K + hv.kv_off, (uint32_t)N * hv.kvs * 2);
  const auto rv = make_rsrc(V + hv.kv_off, (uint32_t)N * hv.kvs * 2);

  bf16x8 qreg[KSTEPS], oreg[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    const uint32_t off = (uint32_t)qrow * (hv.qs * 2) + (16 * kk + 8 * g) * 2;
    qreg[kk] = __builtin_bit_cast(bf16x8, buf_load16(rq, off));
    oreg[kk] = __builtin_bit_cast(bf16x8, buf_load16(rdo, off));
  }
  const float lse2 = (qrow < N) ? LSE[hv.st_off + qrow] * kLog2e : 0.f;
  const float dl = (qrow < N) ? delta[hv.st_off + qrow] : 0.f;  // −D of this row

  f32x16 dq[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[b][r] = 0.f;

  TileDma<D> dma;
  dma.init(wave, lane, hv.kvs);
  TileReads<D> rd0;
  rd0.init(lane);

  const int kv_end = CAUSAL ? min(N, q0 + 128) : N;
  const int ntiles = (kv_end + BC - 1) / BC;
  const int wnt = (qw >= N) ? 0 : (CAUSAL ? min(ntiles, (min(qw + 31, N - 1) / BC) + 1) : ntiles);
  auto issue = [&](int t, bf16* slot) {
    dma.issue(rk, slot, t * BC, hv.kvs);
    dma.issue(rv, slot + TILE, t * BC, hv.kvs);
  };
  issue(0, st0);

  // Operand reads run LOOK products ahead of the product that consumes them
  // (fenced slots keep that order): Sᵀ/dPᵀ products m = 0 .. 4·KSTEPS-1 read
  // K or V rows, then the dQ products read Kᵀ transposed.
  constexpr int LOOK = 2;
  constexpr int NA = 4 * KSTEPS;   // Sᵀ and dPᵀ products
  constexpr int NC = 4 * DBLK;     // dQᵀ products
  auto step = [&](int t, bf16* kt, bf16* next) {
    bf16* const vt = kt + TILE;
    const int k0 = t * BC;
    wait_vm_all();
    __syncthreads();  // tile t resident; tile t-1 consumed by every wave
    if (t + 1 < ntiles) issue(t + 1, next);
    if (k0 + BC > N) {  // tail: K rows past N must be zero for the transposed product
      zero_rows<D>(kt, N - k0, tid);
      __syncthreads();
    }
    if (t >= wnt) return;

    // The lane offsets are re-derived per step (opaque copy) so that only one
    // stage's LDS addresses are live at a time rather than both stages' sets.
    TileReads<D> rd = rd0;
    asm volatile("" : "+v"(rd.rmb), "+v"(rd.rmx), "+v"(rd.trd));
    // product m < NA: key block m / (2 KSTEPS), k-step (m / 2) % KSTEPS, Sᵀ (even m) or dPᵀ (odd m)
    auto a_op = [&](int m) { return rd.row_major((m & 1) ? vt : kt, m / (2 * KSTEPS), (m / 2) % KSTEPS); };
    auto c_op = [&](int m) { return rd.transposed(kt, m % DBLK, m / DBLK); };  // dQ product m: chunk m / DBLK
    const bool need_mask = (CAUSAL && k0 + BC - 1 > qw) || (k0 + BC > N) || (qw + 32 > N);
    f32x16 s[2], dp[2];
    bf16x8 dsb[4];
    // dSᵀ for key block kb, right after its last product: the block's scores
    // die before the next block's accumulate, which keeps two waves per SIMD
    // in registers (the other wave's products cover this one's VALU work)
    auto make_ds = [&](int kb) __attribute__((always_inline)) {
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = exp2_fast(__builtin_fmaf(s[kb][r], scale_log2, -lse2));
        float dsr = pr * (dp[kb][r] + dl);
        if (need_mask) {
          const int ka = k0 + crow(kb, r, g);
          const bool dead = ka >= N || qrow >= N || (CAUSAL && ka > qrow);
          dsr = dead ? 0.f : dsr;
        }
        ds[r] = dsr;
      }
      dsb[2 * kb] = pack8(ds);
      dsb[2 * kb + 1] = pack8(ds + 8);
    };
    bf16x8 op[LOOK + 1];
    static_for<0, LOOK>([&](auto ic) __attribute__((always_inline)) { op[ic.value] = a_op(ic.value); });
    static_for<0, NA>([&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value;
      constexpr int ahead = m + LOOK;
      if constexpr (ahead < NA)
        op[ahead % (LOOK + 1)] = a_op(ahead);
      else
        op[ahead % (LOOK + 1)] = c_op(ahead - NA);
      __builtin_amdgcn_sched_barrier(0);  // the read goes out before this slot's product
      constexpr int kb = m / (2 * KSTEPS), kk = (m / 2) % KSTEPS;
      f32x16& acc = (m & 1) ? dp[kb] : s[kb];
      acc = mfma32(op[m % (LOOK + 1)], (m & 1) ? oreg[kk] : qreg[kk], kk == 0 ? f32x16{} : acc);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (m % (2 * KSTEPS) == 2 * KSTEPS - 1) {
        make_ds(kb);
        __builtin_amdgcn_sched_barrier(0);
      }
    });
    // dQᵀ += Kᵀ dSᵀ
    static_for<0, NC>([&](auto mc) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value;
      constexpr int ahead = NA + m + LOOK;
      if constexpr (ahead < NA + NC) op[ahead % (LOOK + 1)] = c_op(ahead - NA);
      __builtin_amdgcn_sched_barrier(0);
      dq[m % DBLK] = mfma32(op[(NA + m) % (LOOK + 1)], dsb[m / DBLK], dq[m % DBLK]);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  for (int t = 0; t < ntiles; t += 2) {
    step(t, st0, st1);
    if (t + 1 < ntiles) step(t + 1, st1, st0);
  }

  if (qw >= N || qrow >= N) return;
  bf16* row = dQ + hv.q_off + (size_t)qrow * hv.qs;
  const float qs = hv.cut ? kNaN : scale;
#pragma unroll
  for (int b = 0; b < DBLK; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x2 w;
      w[0] = pack_bf16x2(dq[b][4 * i] * qs, dq[b][4 * i + 1] * qs);
      w[1] = pack_bf16x2(dq[b][4 * i + 2] * qs, dq[b][4 * i + 3] * qs);
      *reinterpret_cast<u32x2*>(row + 32 * b + 8 * i + 4 * g) = w;
    }
}

template <int D>
hipError_t launch(const BackwardArgs& a) {
  const bool packed = a.s.cu != nullptr;
  const long long rows = packed ? (long long)a.s.total * a.s.H : (long long)a.s.B * a.s.H * a.s.N;
  constexpr int RPB = kThreads / (D / 8);
  if (rows > 0)
    hipLaunchKernelGGL((bwd_delta_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(kThreads), 0, a.stream,
                       static_cast<const bf16*>(a.o), static_cast<const bf16*>(a.dout), a.lse, a.delta, a.lse2, rows, a.s.H,
                       (long long)a.s.total, packed ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float sl2 = a.scale * kLog2e;
  auto* q = static_cast<const bf16*>(a.q);
  auto* k = static_cast<const bf16*>(a.k);
  auto* v = static_cast<const bf16*>(a.v);
  auto* dout = static_cast<const bf16*>(a.dout);
  const int tiles = (a.s.N + 127) / 128;
  const dim3 grid_kv((unsigned)(tiles * a.s.B * a.s.Hkv)), grid_q((unsigned)(tiles * a.s.B * a.s.H)), block(kThreads);
  if (a.causal) {
    if constexpr (D == 128)
      hipLaunchKernelGGL((bwd_dkdv_pipe_kernel<true>), grid_kv, block, 0, a.stream, q, k, v, dout, a.lse2, a.delta,
                         static_cast<bf16*>(a.dk), static_cast<bf16*>(a.dv), a.s, a.scale, sl2);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, true>), grid_kv, block, 0, a.stream, q, k, v, dout, a.lse, a.delta,
                         static_cast<bf16*>(a.dk), static_cast<bf16*>(a.dv), a.s, a.scale, sl2);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dq_kernel<D, true>), grid_q, block, 0, a.stream, q, k, v, dout, a.lse, a.delta,
                       static_cast<bf16*>(a.dq), a.s, a.scale, sl2);
  } else {
    if constexpr (D == 128)
      hipLaunchKernelGGL((bwd_dkdv_pipe_kernel<false>), grid_kv, block, 0, a.stream, q, k, v, dout, a.lse2, a.delta,
                         static_cast<bf16*>(a.dk), static_cast<bf16*>(a.dv), a.s, a.scale, sl2);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, false>), grid_kv, block, 0, a.stream, q, k, v, dout, a.lse, a.delta,
                         static_cast<bf16*>(a.dk), static_cast<bf16*>(a.dv), a.s, a.scale, sl2);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dq_kernel<D, false>), grid_q, block, 0, a.stream, q, k, v, dout, a.lse, a.delta,
                       static_cast<bf16*>(a.dq), a.s, a.scale, sl2);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const BackwardArgs& a) { return a.d == 128 ? launch<128>(a) : launch<64>(a); }

}  // namespace fa
