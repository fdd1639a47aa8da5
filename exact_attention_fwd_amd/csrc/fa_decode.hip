// Paged split-KV decode for gfx950: one query token per sequence against the
// sequence's KV cache, stored in fixed 256-token pages of a pool and reached
// through a block table (0539edu.com "Flash不是那个被时代淘汰的插件" §2: the
// page pool reserved up front, pages handed to sequences, decode bound by
// cache reads).
//
// Kernel 1 (split): one workgroup per (sequence, page, group of 8 heads).  A
// head's 256-byte K row of one token is read by 16 lanes (16 bytes each), so
// the 8 heads of one token are a contiguous 2 KiB read by two wavefronts.
// Each lane keeps the online-softmax state of its (token parity, head, 8
// features) over blocks of 8 tokens; scores are reduced over the 16 lanes
// with DPP.  The result per (sequence, head, page) is the partial running
// max, normaliser and unnormalised output.
// Kernel 2 (merge): combines the partials of a (sequence, head) exactly:
// m = max m_b, l = Σ 2^(m_b − m) l_b, O = Σ 2^(m_b − m) õ_b / l — the running
// max / normaliser update of "Flash Attention 是什么" (ai.lansai.wang),
// 关键术语解析 §4, applied to partial states instead of single blocks.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kDecThreads = 256;
constexpr int kPage = 256;
constexpr int kUnroll = 8;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of LPR (8 or 16) lanes; every lane gets the total.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  x += dpp<0x141>(x);  // row_half_mirror: pairs the two quads of 8 lanes
  if (LPR == 16) x += dpp<0x140>(x);  // row_mirror: pairs the two halves of 16 lanes
  return x;
}

__device__ __forceinline__ void bf16x8_to_f32(const u32x4& w, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <int D, int HG>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ pool, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, float* __restrict__ part, int H, int max_blocks, float scale_log2) {
  constexpr int LPR = D / 8;                       // lanes per (token, head) row
  constexpr int TP = kDecThreads / (HG * LPR);     // tokens handled side by side
  constexpr int STEPS = kPage / TP;                // tokens per lane in one page
  static_assert(STEPS % kUnroll == 0, "page must split evenly");
  __shared__ float red[TP][HG][D + 2];

  const int hgroups = H / HG;
  const int s = blockIdx.x / (max_blocks * hgroups);
  const int rem = blockIdx.x % (max_blocks * hgroups);
  const int b = rem / hgroups;
  const int h0 = (rem % hgroups) * HG;
  const int L = seq_lens[s];
  const int ntok = min(kPage, L - b * kPage);
  if (ntok <= 0) return;  // this page is past the sequence end
  const int page = block_table[(size_t)s * max_blocks + b];

  const int tid = threadIdx.x;
  const int c = tid % LPR;
  const int hh = (tid / LPR) % HG;
  const int tp = tid / (LPR * HG);
  const int h = h0 + hh;

  float qf[8];
  bf16x8_to_f32(*reinterpret_cast<const u32x4*>(q + ((size_t)s * H + h) * D + c * 8), qf);
#pragma unroll
  for (int e = 0; e < 8; ++e) qf[e] *= scale_log2;

  const size_t tok_stride = (size_t)H * D;
  const bf16* Kp = pool + (size_t)page * 2 * kPage * tok_stride + (size_t)h * D + c * 8;
  const bf16* Vp = Kp + (size_t)kPage * tok_stride;

  float m = kNegInf, l = 0.f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;

  for (int i0 = 0; i0 < STEPS; i0 += kUnroll) {
    u32x4 kr[kUnroll], vr[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = tp + TP * (i0 + u);
      const bool ok = t < ntok;
      u32x4 zero = {0u, 0u, 0u, 0u};
      kr[u] = ok ? *reinterpret_cast<const u32x4*>(Kp + t * tok_stride) : zero;
      vr[u] = ok ? *reinterpret_cast<const u32x4*>(Vp + t * tok_stride) : zero;
    }
    float sc[kUnroll];
    float bmax = kNegInf;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float kf[8];
      bf16x8_to_f32(kr[u], kf);
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(qf[e], kf[e], acc);
      acc = group_sum<LPR>(acc);
      const int t = tp + TP * (i0 + u);
      sc[u] = (t < ntok) ? acc : kNegInf;
      bmax = fmaxf(bmax, sc[u]);
    }
    if (bmax == kNegInf) continue;  // every token of this block is past the end
    const float m_new = fmaxf(m, bmax);
    const float alpha = exp2_fast(m - m_new);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= alpha;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float p = exp2_fast(sc[u] - m_new);  // 0 for tokens past the end
      l += p;
      float vf[8];
      bf16x8_to_f32(vr[u], vf);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = __builtin_fmaf(p, vf[e], o[e]);
    }
    m = m_new;
  }

  // Merge the TP token streams of each (head, feature chunk) through LDS.
  float* mine = red[tp][hh];
#pragma unroll
  for (int e = 0; e < 8; ++e) mine[c * 8 + e] = o[e];
  if (c == 0) {
    mine[D] = m;
    mine[D + 1] = l;
  }
  __syncthreads();
  if (tp != 0) return;
  float mm = kNegInf;
#pragma unroll
  for (int j = 0; j < TP; ++j) mm = fmaxf(mm, red[j][hh][D]);
  float ll = 0.f, oo[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) oo[e] = 0.f;
#pragma unroll
  for (int j = 0; j < TP; ++j) {
    const float mj = red[j][hh][D];
    const float w = (mj == kNegInf) ? 0.f : exp2_fast(mj - mm);
    ll += w * red[j][hh][D + 1];
#pragma unroll
    for (int e = 0; e < 8; ++e) oo[e] += w * red[j][hh][c * 8 + e];
  }
  float* out = part + (((size_t)s * H + h) * max_blocks + b) * (D + 2);
#pragma unroll
  for (int e = 0; e < 8; ++e) out[c * 8 + e] = oo[e];
  if (c == 0) {
    out[D] = mm;
    out[D + 1] = ll;
  }
}

// One wavefront per (sequence, head): merge the per-page partial states.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(const float* __restrict__ part,
                                                          const int32_t* __restrict__ seq_lens,
                                                          bf16* __restrict__ O, float* __restrict__ LSE, int H,
                                                          int max_blocks) {
  constexpr int PER = D / 64;
  const int sh = blockIdx.x;
  const int s = sh / H;
  const int lane = threadIdx.x;
  const int nb = (seq_lens[s] + kPage - 1) / kPage;
  const float* p = part + (size_t)sh * max_blocks * (D + 2);
  float m = kNegInf;
  for (int b = 0; b < nb; ++b) m = fmaxf(m, p[(size_t)b * (D + 2) + D]);
  float l = 0.f, o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
  for (int b = 0; b < nb; ++b) {
    const float* pb = p + (size_t)b * (D + 2);
    const float w = exp2_fast(pb[D] - m);
    l += w * pb[D + 1];
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] += w * pb[lane * PER + e];
  }
  const float inv = 1.f / l;
  bf16* orow = O + (size_t)sh * D;
#pragma unroll
  for (int e = 0; e < PER; ++e) orow[lane * PER + e] = (bf16)(o[e] * inv);
  if (LSE != nullptr && lane == 0) LSE[sh] = (m + log2_fast(l)) * kLn2;
}

template <int D, int HG>
hipError_t launch(const DecodeArgs& a) {
  const int hgroups = a.H / HG;
  const dim3 grid1((unsigned)(a.S * a.max_blocks * hgroups)), block1(kDecThreads);
  hipLaunchKernelGGL((decode_split_kernel<D, HG>), grid1, block1, 0, a.stream, static_cast<const bf16*>(a.q),
                     static_cast<const bf16*>(a.kv_pool), a.block_table, a.seq_lens, a.part, a.H, a.max_blocks,
                     a.scale * kLog2e);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(a.S * a.H), dim3(64), 0, a.stream, a.part, a.seq_lens,
                     static_cast<bf16*>(a.o), a.lse, a.H, a.max_blocks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a) {
  if (a.d == 128) return (a.H % 8 == 0) ? launch<128, 8>(a) : launch<128, 1>(a);
  return (a.H % 8 == 0) ? launch<64, 8>(a) : launch<64, 1>(a);
}

}  // namespace fa
