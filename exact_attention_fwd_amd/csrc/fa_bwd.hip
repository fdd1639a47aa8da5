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
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_delta_kernel(const bf16* __restrict__ O, const bf16* __restrict__ dO,
                                                             float* __restrict__ delta, long long rows) {
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
  if (row < rows && c == 0) delta[row] = acc;
}

// ---------------------------------------------------------------------------
// dK, dV: workgroup = 128 keys of one head; wavefront w owns keys kw..kw+31.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ delta,
    bf16* __restrict__ dK, bf16* __restrict__ dV, int N, float scale, float scale_log2) {
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int BQ = kTileRows;  // queries per step
  __shared__ __attribute__((aligned(16))) bf16 sQ[BQ * D];
  __shared__ __attribute__((aligned(16))) bf16 sQt[D * BQ];
  __shared__ __attribute__((aligned(16))) bf16 sdO[BQ * D];
  __shared__ __attribute__((aligned(16))) bf16 sdOt[D * BQ];
  __shared__ __attribute__((aligned(16))) float sL[BQ];
  __shared__ __attribute__((aligned(16))) float sDl[BQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, n = lane & 31;
  const int bh = blockIdx.y;
  const int k0 = blockIdx.x * 128;
  const int kw = k0 + 32 * wave;
  const int key = kw + n;  // this lane's key column
  const bool wave_live = kw < N;
  const size_t head_off = (size_t)bh * N * D;
  const bf16* Qh = Q + head_off;
  const bf16* dOh = dO + head_off;
  const float* Lh = LSE + (size_t)bh * N;
  const float* Dh = delta + (size_t)bh * N;

  // Kᵀ and Vᵀ as B operands: lane (g, n) holds row `key`, features 16kk+8g..
  bf16x8 kreg[KSTEPS], vreg[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
    if (key < N) {
      x = *reinterpret_cast<const u32x4*>(K + head_off + (size_t)key * D + 16 * kk + 8 * g);
      y = *reinterpret_cast<const u32x4*>(V + head_off + (size_t)key * D + 16 * kk + 8 * g);
    }
    kreg[kk] = __builtin_bit_cast(bf16x8, x);
    vreg[kk] = __builtin_bit_cast(bf16x8, y);
  }
  f32x16 dk[DBLK], dv[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[b][r] = 0.f;
      dv[b][r] = 0.f;
    }

  const int qstart = CAUSAL ? (k0 / BQ) * BQ : 0;
  for (int q0 = qstart; q0 < N; q0 += BQ) {
    __syncthreads();
    {
      RowTile<D, kThreads> t;
      t.load(Qh, q0, N, tid);
      t.store(sQ, tid);
      t.load(dOh, q0, N, tid);
      t.store(sdO, tid);
      TransTile<D, kThreads> u;
      u.load(Qh, q0, N, tid);
      u.store(sQt, tid);
      u.load(dOh, q0, N, tid);
      u.store(sdOt, tid);
      if (tid < BQ) {
        const bool ok = q0 + tid < N;
        sL[tid] = ok ? Lh[q0 + tid] * kLog2e : 0.f;
        sDl[tid] = ok ? Dh[q0 + tid] : 0.f;
      }
    }
    __syncthreads();
    if (!wave_live || (CAUSAL && q0 + BQ - 1 < kw)) continue;
    const bool need_mask = (CAUSAL && q0 < kw + 31) || (q0 + BQ > N) || (kw + 32 > N);

#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      // S = Q Kᵀ and dP = dO Vᵀ for 32 queries (rows) x this lane's key.
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
      const int row = 32 * qb + perm_row(n);
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        s = mfma32(lds_rm_read<D>(sQ, row, 2 * kk + g), kreg[kk], s);
        dp = mfma32(lds_rm_read<D>(sdO, row, 2 * kk + g), vreg[kk], dp);
      }
      float p[16], ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = crow(qb, r, g);
        float pr = exp2_fast(__builtin_fmaf(s[r], scale_log2, -sL[qi]));
        if (need_mask) {
          const int qa = q0 + qi;
          const bool dead = qa >= N || key >= N || (CAUSAL && key > qa);
          pr = dead ? 0.f : pr;
        }
        p[r] = pr;
        ds[r] = pr * (dp[r] - sDl[qi]);
      }
      const bf16x8 p0 = pack8(p), p1 = pack8(p + 8);
      const bf16x8 d0 = pack8(ds), d1 = pack8(ds + 8);
      // dVᵀ += dOᵀ P ; dKᵀ += Qᵀ dS   (k-steps over this block's 32 queries)
#pragma unroll
      for (int b = 0; b < DBLK; ++b) {
        const int d = 32 * b + n;
        dv[b] = mfma32(lds_tr_read(sdOt, d, 4 * qb + g), p0, dv[b]);
        dv[b] = mfma32(lds_tr_read(sdOt, d, 4 * qb + 2 + g), p1, dv[b]);
        dk[b] = mfma32(lds_tr_read(sQt, d, 4 * qb + g), d0, dk[b]);
        dk[b] = mfma32(lds_tr_read(sQt, d, 4 * qb + 2 + g), d1, dk[b]);
      }
    }
  }

  if (!wave_live || key >= N) return;
  bf16* dKrow = dK + head_off + (size_t)key * D;
  bf16* dVrow = dV + head_off + (size_t)key * D;
#pragma unroll
  for (int b = 0; b < DBLK; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x2 wk, wv;
      wk[0] = pack_bf16x2(dk[b][4 * i] * scale, dk[b][4 * i + 1] * scale);
      wk[1] = pack_bf16x2(dk[b][4 * i + 2] * scale, dk[b][4 * i + 3] * scale);
      wv[0] = pack_bf16x2(dv[b][4 * i], dv[b][4 * i + 1]);
      wv[1] = pack_bf16x2(dv[b][4 * i + 2], dv[b][4 * i + 3]);
      *reinterpret_cast<u32x2*>(dKrow + 32 * b + 8 * i + 4 * g) = wk;
      *reinterpret_cast<u32x2*>(dVrow + 32 * b + 8 * i + 4 * g) = wv;
    }
}

// ---------------------------------------------------------------------------
// dQ: workgroup = 128 queries of one head; wavefront w owns qw..qw+31.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void bwd_dq_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ delta,
    bf16* __restrict__ dQ, int N, float scale, float scale_log2) {
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int BC = kTileRows;
  __shared__ __attribute__((aligned(16))) bf16 sK[BC * D];
  __shared__ __attribute__((aligned(16))) bf16 sKt[D * BC];
  __shared__ __attribute__((aligned(16))) bf16 sV[BC * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, n = lane & 31;
  const int bh = blockIdx.y;
  const int nqb = (N + 127) / 128;
  const int qblk = CAUSAL ? (nqb - 1 - (int)blockIdx.x) : (int)blockIdx.x;  // heavy tiles first
  const int q0 = qblk * 128;
  const int qw = q0 + 32 * wave;
  const int qrow = qw + n;
  const bool wave_live = qw < N;
  const size_t head_off = (size_t)bh * N * D;
  const bf16* Kh = K + head_off;
  const bf16* Vh = V + head_off;

  bf16x8 qreg[KSTEPS], oreg[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
    if (qrow < N) {
      x = *reinterpret_cast<const u32x4*>(Q + head_off + (size_t)qrow * D + 16 * kk + 8 * g);
      y = *reinterpret_cast<const u32x4*>(dO + head_off + (size_t)qrow * D + 16 * kk + 8 * g);
    }
    qreg[kk] = __builtin_bit_cast(bf16x8, x);
    oreg[kk] = __builtin_bit_cast(bf16x8, y);
  }
  const float lse2 = (qrow < N) ? LSE[(size_t)bh * N + qrow] * kLog2e : 0.f;
  const float dl = (qrow < N) ? delta[(size_t)bh * N + qrow] : 0.f;

  f32x16 dq[DBLK];
#pragma unroll
  for (int b = 0; b < DBLK; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[b][r] = 0.f;

  const int kv_end = CAUSAL ? min(N, q0 + 128) : N;
  for (int k0 = 0; k0 < kv_end; k0 += BC) {
    __syncthreads();
    {
      RowTile<D, kThreads> t;
      t.load(Kh, k0, N, tid);
      t.store(sK, tid);
      t.load(Vh, k0, N, tid);
      t.store(sV, tid);
      TransTile<D, kThreads> u;
      u.load(Kh, k0, N, tid);
      u.store(sKt, tid);
    }
    __syncthreads();
    if (!wave_live || (CAUSAL && k0 > qw + 31)) continue;
    const bool need_mask = (CAUSAL && k0 + BC - 1 > qw) || (k0 + BC > N) || (qw + 32 > N);

    bf16x8 dsb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
      const int row = 32 * kb + perm_row(n);
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        s = mfma32(lds_rm_read<D>(sK, row, 2 * kk + g), qreg[kk], s);
        dp = mfma32(lds_rm_read<D>(sV, row, 2 * kk + g), oreg[kk], dp);
      }
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pr = exp2_fast(__builtin_fmaf(s[r], scale_log2, -lse2));
        if (need_mask) {
          const int ka = k0 + crow(kb, r, g);
          const bool dead = ka >= N || qrow >= N || (CAUSAL && ka > qrow);
          pr = dead ? 0.f : pr;
        }
        ds[r] = pr * (dp[r] - dl);
      }
      dsb[2 * kb] = pack8(ds);
      dsb[2 * kb + 1] = pack8(ds + 8);
    }
    // dQᵀ += Kᵀ dSᵀ
#pragma unroll
    for (int b = 0; b < DBLK; ++b) {
      const int d = 32 * b + n;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) dq[b] = mfma32(lds_tr_read(sKt, d, 2 * kk + g), dsb[kk], dq[b]);
    }
  }

  if (!wave_live || qrow >= N) return;
  bf16* row = dQ + head_off + (size_t)qrow * D;
#pragma unroll
  for (int b = 0; b < DBLK; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x2 w;
      w[0] = pack_bf16x2(dq[b][4 * i] * scale, dq[b][4 * i + 1] * scale);
      w[1] = pack_bf16x2(dq[b][4 * i + 2] * scale, dq[b][4 * i + 3] * scale);
      *reinterpret_cast<u32x2*>(row + 32 * b + 8 * i + 4 * g) = w;
    }
}

template <int D>
hipError_t launch(const BackwardArgs& a) {
  const long long rows = (long long)a.BH * a.N;
  constexpr int RPB = kThreads / (D / 8);
  hipLaunchKernelGGL((bwd_delta_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(kThreads), 0, a.stream,
                     static_cast<const bf16*>(a.o), static_cast<const bf16*>(a.dout), a.delta, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float sl2 = a.scale * kLog2e;
  auto* q = static_cast<const bf16*>(a.q);
  auto* k = static_cast<const bf16*>(a.k);
  auto* v = static_cast<const bf16*>(a.v);
  auto* dout = static_cast<const bf16*>(a.dout);
  const dim3 grid((a.N + 127) / 128, a.BH), block(kThreads);
  if (a.causal) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, true>), grid, block, 0, a.stream, q, k, v, dout, a.lse, a.delta,
                       static_cast<bf16*>(a.dk), static_cast<bf16*>(a.dv), a.N, a.scale, sl2);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dq_kernel<D, true>), grid, block, 0, a.stream, q, k, v, dout, a.lse, a.delta,
                       static_cast<bf16*>(a.dq), a.N, a.scale, sl2);
  } else {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, false>), grid, block, 0, a.stream, q, k, v, dout, a.lse, a.delta,
                       static_cast<bf16*>(a.dk), static_cast<bf16*>(a.dv), a.N, a.scale, sl2);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dq_kernel<D, false>), grid, block, 0, a.stream, q, k, v, dout, a.lse, a.delta,
                       static_cast<bf16*>(a.dq), a.N, a.scale, sl2);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const BackwardArgs& a) { return a.d == 128 ? launch<128>(a) : launch<64>(a); }

}  // namespace fa
