// Fused exact-attention forward for gfx950.
//
// One workgroup owns a tile of 128 queries of one (batch, head); each of its
// four wavefronts owns 32 of those queries.  Key/value tiles of 64 tokens are
// streamed through LDS (K row-major, V transposed), and per tile a wave
//   1. computes Sᵀ = K·Qᵀ (64 keys x 32 queries) on bf16 MFMA, Q kept in
//      registers for the whole pass,
//   2. masks future keys (diagonal tiles only) and keys past N,
//   3. runs the online softmax: new running max, rescale factor for the old
//      partial output and normaliser, p = 2^(s·scale·log2e − m),
//   4. rounds p to bf16 and accumulates Oᵀ += Vᵀ·Pᵀ on MFMA.
// Holding Sᵀ (one query per lane) keeps every row reduction inside a lane
// plus one exchange with lane ^ 32, and makes the rescale of O a per-lane
// scalar.  Only O (bf16, round-to-nearest-even) and the natural-log
// logsumexp are written back; no score tile ever reaches device memory.
//
// Method: "Flash Attention 是什么：2026 最新原理、架构演进与实战详解"
// (ai.lansai.wang), 技术原理 › 核心工作机制 (tiling into on-chip memory and
// the online softmax) and 关键术语解析 §4 (the running max m and normaliser l
// updates); zwxr.cn §3.1 (rescale by the final normaliser once at the end).
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kBR = 128;  // queries per workgroup
constexpr int kBC = 64;   // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// Map the linear block id to (query tile, batch*head).  Blocks are handed out
// round-robin over the 8 XCDs, so the ids of one XCD are bid % 8 == x.  Heads
// are grouped per XCD (their K/V then share that XCD's L2), and within an
// XCD the query tiles with the most work (causal: the last ones) go first.
__device__ __forceinline__ void map_block(int bid, int nqb, int BH, bool causal, int& qb, int& bh) {
  const int total = nqb * BH;
  int rank, head;
  if ((BH & 7) == 0) {
    const int xcd = bid & 7, slot = bid >> 3;
    const int hpx = BH >> 3;
    rank = slot / hpx;
    head = xcd * hpx + slot % hpx;
  } else {
    rank = bid / BH;
    head = bid % BH;
  }
  (void)total;
  qb = causal ? (nqb - 1 - rank) : rank;
  bh = head;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, int N, int BH, float scale_log2) {
  constexpr int KSTEPS = D / 16;  // MFMA k-steps over the head dim
  constexpr int DBLK = D / 32;    // 32-row output blocks over the head dim
  __shared__ __attribute__((aligned(16))) bf16 sK[kTileRows * D];
  __shared__ __attribute__((aligned(16))) bf16 sVt[D * kTileRows];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, n = lane & 31;
  const int nqb = (N + kBR - 1) / kBR;
  int qb, bh;
  map_block(blockIdx.x, nqb, BH, CAUSAL, qb, bh);

  const size_t head_off = (size_t)bh * N * D;
  const bf16* Qh = Q + head_off;
  const bf16* Kh = K + head_off;
  const bf16* Vh = V + head_off;
  const int q0 = qb * kBR;
  const int qw = q0 + wave * 32;
  const int qrow = qw + n;  // this lane's query
  const bool wave_live = qw < N;

  // Qᵀ as the B operand: lane (g, n) holds Q[qrow][16kk + 8g .. +7].
  bf16x8 qreg[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (qrow < N) x = *reinterpret_cast<const u32x4*>(Qh + (size_t)qrow * D + 16 * kk + 8 * g);
    qreg[kk] = __builtin_bit_cast(bf16x8, x);
  }

  f32x16 oacc[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[b][r] = 0.f;
  float m_run = kNegInf;  // running max of s·scale·log2e
  float l_run = 0.f;      // this lane's part of the running normaliser

  const int kv_end = CAUSAL ? min(N, q0 + kBR) : N;
  const int ntiles = (kv_end + kBC - 1) / kBC;

  RowTile<D, kThreads> kt;
  TransTile<D, kThreads> vt;
  kt.load(Kh, 0, N, tid);
  vt.load(Vh, 0, N, tid);

  for (int t = 0; t < ntiles; ++t) {
    const int k0 = t * kBC;
    __syncthreads();  // every wave is done reading the previous tile
    kt.store(sK, tid);
    vt.store(sVt, tid);
    __syncthreads();
    if (t + 1 < ntiles) {  // prefetch the next tile while this one is consumed
      kt.load(Kh, k0 + kBC, N, tid);
      vt.load(Vh, k0 + kBC, N, tid);
    }
    if (!wave_live || (CAUSAL && k0 > qw + 31)) continue;

    // ---- Sᵀ = K Qᵀ : two 32-key blocks -------------------------------------
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
      const int row = 32 * kb + perm_row(n);
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) s[kb] = mfma32(lds_rm_read<D>(sK, row, 2 * kk + g), qreg[kk], s[kb]);
    }

    // ---- mask: future keys (causal diagonal) and keys past N ----------------
    const bool need_mask = (CAUSAL && k0 + kBC - 1 > qw) || (k0 + kBC > N);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + crow(kb, r, g);
          const bool dead = (key >= N) || (CAUSAL && key > qrow);
          s[kb][r] = dead ? kNegInf : s[kb][r];
        }
    }

    // ---- online softmax ------------------------------------------------------
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = xhalf_max(mx);
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = exp2_fast(m_run - m_use);
    float psum = 0.f;
    bf16x8 pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          p[j] = exp2_fast(__builtin_fmaf(s[kb][8 * h + j], scale_log2, -m_use));
          psum += p[j];
        }
        pb[2 * kb + h] = pack8(p);
      }
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int b = 0; b < DBLK; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[b][r] *= alpha;

    // ---- Oᵀ += Vᵀ Pᵀ -----------------------------------------------------------
#pragma unroll
    for (int b = 0; b < DBLK; ++b) {
      const int d = 32 * b + n;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) oacc[b] = mfma32(lds_tr_read(sVt, d, 2 * kk + g), pb[kk], oacc[b]);
    }
  }

  if (!wave_live || qrow >= N) return;
  const float l_tot = xhalf_sum(l_run);
  const float inv = 1.f / l_tot;
  bf16* Orow = O + head_off + (size_t)qrow * D;
#pragma unroll
  for (int b = 0; b < DBLK; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x2 w;
      w[0] = pack_bf16x2(oacc[b][4 * i + 0] * inv, oacc[b][4 * i + 1] * inv);
      w[1] = pack_bf16x2(oacc[b][4 * i + 2] * inv, oacc[b][4 * i + 3] * inv);
      *reinterpret_cast<u32x2*>(Orow + 32 * b + 8 * i + 4 * g) = w;
    }
  if (LSE != nullptr && g == 0) LSE[(size_t)bh * N + qrow] = (m_run + log2_fast(l_tot)) * kLn2;
}

// fp32 path: one thread per query row, keys staged through LDS 32 at a time,
// fp32 fused multiply-adds and an online softmax updated key by key.
template <int D>
__global__ __launch_bounds__(64) void fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                     const float* __restrict__ V, float* __restrict__ O,
                                                     float* __restrict__ LSE, int N, float scale, int causal) {
  constexpr int TK = 32;
  __shared__ float sk[TK][D];
  __shared__ float sv[TK][D];
  const int tid = threadIdx.x;
  const int row = blockIdx.x * 64 + tid;
  const size_t head_off = (size_t)blockIdx.y * N * D;
  float q[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = row < N ? Q[head_off + (size_t)row * D + d] : 0.f;
    acc[d] = 0.f;
  }
  float m = kNegInf, l = 0.f;
  const int kend = causal ? min(N, (int)blockIdx.x * 64 + 64) : N;
  for (int k0 = 0; k0 < kend; k0 += TK) {
    __syncthreads();
    for (int i = tid; i < TK * D; i += 64) {
      const int r = i / D, d = i % D;
      const bool ok = k0 + r < N;
      sk[r][d] = ok ? K[head_off + (size_t)(k0 + r) * D + d] : 0.f;
      sv[r][d] = ok ? V[head_off + (size_t)(k0 + r) * D + d] : 0.f;
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
  const float inv = 1.f / l;
#pragma unroll
  for (int d = 0; d < D; ++d) O[head_off + (size_t)row * D + d] = acc[d] * inv;
  if (LSE != nullptr) LSE[(size_t)blockIdx.y * N + row] = m + logf(l);
}

template <int D>
hipError_t launch_bf16(const ForwardArgs& a) {
  const int nqb = (a.N + kBR - 1) / kBR;
  const dim3 grid(nqb * a.BH), block(kThreads);
  const float sl2 = a.scale * kLog2e;
  auto* q = static_cast<const bf16*>(a.q);
  auto* k = static_cast<const bf16*>(a.k);
  auto* v = static_cast<const bf16*>(a.v);
  auto* o = static_cast<bf16*>(a.o);
  if (a.causal)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, true>), grid, block, 0, a.stream, q, k, v, o, a.lse, a.N, a.BH, sl2);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, false>), grid, block, 0, a.stream, q, k, v, o, a.lse, a.N, a.BH, sl2);
  return hipGetLastError();
}

template <int D>
hipError_t launch_f32(const ForwardArgs& a) {
  const dim3 grid((a.N + 63) / 64, a.BH), block(64);
  hipLaunchKernelGGL((fwd_f32_kernel<D>), grid, block, 0, a.stream, static_cast<const float*>(a.q),
                     static_cast<const float*>(a.k), static_cast<const float*>(a.v), static_cast<float*>(a.o),
                     a.lse, a.N, a.scale, a.causal);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward(const ForwardArgs& a) {
  if (a.bf16) return a.d == 128 ? launch_bf16<128>(a) : launch_bf16<64>(a);
  return a.d == 128 ? launch_f32<128>(a) : launch_f32<64>(a);
}

}  // namespace fa
