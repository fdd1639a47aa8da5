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
// features) over blocks of 8 tokens.  Scores are bf16 dot products
// (v_dot2_f32_bf16, fp32 accumulate) reduced over the 16 lanes with DPP;
// p·V runs as dot2 over token pairs.  K/V are read through buffer
// descriptors that end at the sequence's last token, so slots past it are
// never fetched.  The result per (sequence, head, page) is the partial
// running max, normaliser and unnormalised output.
// Kernel 1' (split, grouped key/value heads): the g = H / Hkv query heads
// that share a key/value head read each K/V row once.  Each wavefront works
// alone on one (sequence, split, key/value head, block of up to 32 of its
// query heads), the split being a whole page when the block table is large
// enough to fill the chip that way and half a page otherwise, and streams
// the split in 32-token tiles.  Tile loads read
// whole token rows (16 lanes per 256-byte row, so every cache line fetched
// is used by one instruction) into staging registers; at the start of a tile
// they move to the wave's own K and V tiles in LDS and the registers take the
// next tile's loads.  Sᵀ = K·Qᵀ runs on bf16 MFMA with the group's queries as
// the 32 columns and K rows read back from LDS in operand layout; the
// per-head online softmax is then a column reduction inside a lane pair, and
// Oᵀ += Vᵀ·Pᵀ reads Vᵀ transposed out of LDS.  One partial per (sequence,
// query head, split).
// Multi-query / grouped-query sharing of K/V is the adaptation named by
// "Flash Attention 是什么" (ai.lansai.wang), 进阶学习路径 §4.
// Kernel 2 (merge): combines the partials of a (sequence, head) exactly:
// m = max m_b, l = Σ 2^(m_b − m) l_b, O = Σ 2^(m_b − m) õ_b / l — the running
// max / normaliser update of "Flash Attention 是什么" (ai.lansai.wang),
// 关键术语解析 §4, applied to partial states instead of single blocks.
#include <mutex>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

// Device-resident scratch for callers that cannot allocate (the decode
// partials of fa_decode_paged_gqa_static).  Each GPU the library runs on
// holds its own copy, zero-filled when the code object loads, until the
// process ends.  Host code never names this array directly: its name is a
// host-side stand-in, so kernels get the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kDecThreads = 256;
constexpr int kPage = 256;
constexpr int kSplit = 128;                 // tokens per workgroup (two splits per page)
constexpr int kSplitsPerPage = kPage / kSplit;
constexpr int kUnroll = 8;                  // tokens per lane per load batch

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

// Rescale the partial output only when the running max grows by more than
// 2^8 (same reference max for output, normaliser and logsumexp: exact).
constexpr float kRescaleThreshold = 8.0f;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

template <int D, int HG>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ pool, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, float* __restrict__ part, int H, int num_pages, int max_blocks,
    float scale_log2) {
  constexpr int LPR = D / 8;                       // lanes per (token, head) row
  constexpr int TP = kDecThreads / (HG * LPR);     // tokens handled side by side
  constexpr int STEPS = kSplit / TP;               // tokens per lane in one split
  constexpr int U = (STEPS / 2 < kUnroll) ? STEPS / 2 : kUnroll;  // tokens per lane per batch
  static_assert(STEPS % (2 * U) == 0 && U % 2 == 0, "split must divide into pairs of batches");
  __shared__ float red[TP][HG][D + 2];

  const int hgroups = H / HG;
  const int nsplit = max_blocks * kSplitsPerPage;
  const int s = blockIdx.x / (nsplit * hgroups);
  const int rem = blockIdx.x % (nsplit * hgroups);
  const int sp = rem / hgroups;                    // split index within the sequence
  const int h0 = (rem % hgroups) * HG;
  const int b = sp / kSplitsPerPage;               // logical page
  const int t0 = (sp % kSplitsPerPage) * kSplit;   // first slot of this split in the page
  const int L = seq_lens[s];
  const int ntok = min(kSplit, L - b * kPage - t0);
  if (ntok <= 0) return;  // this split is past the sequence end
  // (a table entry outside the pool is clamped into it: never an access outside the pool)
  const int page = min(max(block_table[(size_t)s * max_blocks + b], 0), num_pages - 1);

  const int tid = threadIdx.x;
  const int c = tid % LPR;
  const int hh = (tid / LPR) % HG;
  const int tp = tid / (LPR * HG);
  const int h = h0 + hh;

  // This lane's 8 query features, packed bf16 pairs (exact input values).
  const u32x4 qv = *reinterpret_cast<const u32x4*>(q + ((size_t)s * H + h) * D + c * 8);

  // K and V of this split as bounds-checked buffers covering exactly its
  // valid tokens: a slot at or past L reads as zero and is never fetched.
  const uint32_t tok_bytes = (uint32_t)H * D * 2;
  const bf16* kbase = pool + (size_t)page * 2 * kPage * H * D + (size_t)t0 * H * D;
  const auto rk = make_rsrc(kbase, (uint32_t)ntok * tok_bytes);
  const auto rv = make_rsrc(kbase + (size_t)kPage * H * D, (uint32_t)ntok * tok_bytes);
  const uint32_t lane_off = (uint32_t)(h * D + c * 8) * 2;

  float m = kNegInf, l = 0.f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;

  auto load = [&](int i0, u32x4* kr, u32x4* vr) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t off = (uint32_t)(tp + TP * (i0 + u)) * tok_bytes + lane_off;
      kr[u] = buf_load16_stream(rk, off);
      vr[u] = buf_load16_stream(rv, off);
    }
  };
  auto consume = [&](int i0, const u32x4* kr, const u32x4* vr) {
    float sc[U];
    float bmax = kNegInf;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float acc = dot2(qv[0], kr[u][0], 0.f);
      acc = dot2(qv[1], kr[u][1], acc);
      acc = dot2(qv[2], kr[u][2], acc);
      acc = dot2(qv[3], kr[u][3], acc);
      acc = group_sum<LPR>(acc) * scale_log2;
      sc[u] = (tp + TP * (i0 + u) < ntok) ? acc : kNegInf;
      bmax = fmaxf(bmax, sc[u]);
    }
    if (bmax > m + kRescaleThreshold) {  // uniform over the 16-lane row group
      const float alpha = exp2_fast(m - bmax);
      l *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] *= alpha;
      m = bmax;
    }
    // o += p·v over token pairs: p packed to bf16, v regrouped into
    // (token u, token u+1) pairs per feature, one dot2 per feature pair.
    // A stream that has seen no valid token yet keeps m = -inf; its p are 0.
    const float m_use = (m == kNegInf) ? 0.f : m;
#pragma unroll
    for (int u = 0; u < U; u += 2) {
      const float p0 = exp2_fast(sc[u] - m_use), p1 = exp2_fast(sc[u + 1] - m_use);
      l += p0 + p1;
      const uint32_t pp = pack_bf16x2(p0, p1);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t lo = __builtin_amdgcn_perm(vr[u + 1][w], vr[u][w], 0x05040100u);  // (v_u[2w],   v_u+1[2w])
        const uint32_t hi = __builtin_amdgcn_perm(vr[u + 1][w], vr[u][w], 0x07060302u);  // (v_u[2w+1], v_u+1[2w+1])
        o[2 * w] = dot2(pp, lo, o[2 * w]);
        o[2 * w + 1] = dot2(pp, hi, o[2 * w + 1]);
      }
    }
  };

  // Two register batches: the next batch's loads are in flight while the
  // current one is consumed.
  u32x4 ka[U], va[U], kb2[U], vb2[U];
  load(0, ka, va);
  for (int i0 = 0; i0 < STEPS; i0 += 2 * U) {
    load(i0 + U, kb2, vb2);
    consume(i0, ka, va);
    if (i0 + 2 * U < STEPS) load(i0 + 2 * U, ka, va);
    consume(i0 + U, kb2, vb2);
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
  float* out = part + (((size_t)s * H + h) * nsplit + sp) * (D + 2);
#pragma unroll
  for (int e = 0; e < 8; ++e) out[c * 8 + e] = oo[e];
  if (c == 0) {
    out[D] = mm;
    out[D + 1] = ll;
  }
}

// Query heads per wavefront of the grouped kernel (the MFMA's 32 columns).
constexpr int kGqaCols = 32;
// Tokens per wavefront: a whole page when the grid is large enough to fill
// the chip with pages (fewer partials to merge, longer streams per
// wavefront), half a page otherwise.
constexpr int kGqaPageUnits = 1024;
constexpr int kGqaTile = 32;     // tokens per streamed tile

// Swizzle of the K tile in LDS: 16-byte chunk c of tile row r sits at
// position c ^ k_swz(r).  The rows are read back as an MFMA operand, lane n
// (of 32) taking row perm_row(n), so the swizzle is a function of n: with
// d = 128 (16 chunks per 256-byte row) the 16 lanes of a read hit 16
// distinct chunk positions, with d = 64 (two rows per 256 bytes) the pairs
// (row parity, position) are distinct; in both cases every 8 consecutive
// lanes also differ modulo 128 bytes.  Writes (16 lanes along one row) are
// free of conflicts for any swizzle.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  const int n = perm_row(row);
  return D >= 128 ? (n & 15) : ((n & 7) ^ ((n >> 3) & 1));
}

template <int D, int TPW>
__global__ __launch_bounds__(kDecThreads, 2) void decode_gqa_split_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ pool, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, float* __restrict__ part, int S, int H, int Hkv, int num_pages,
    int max_blocks, float scale_log2) {
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int CPR = D / 8;                  // 16-byte chunks per row
  constexpr int RPL = 64 / CPR;               // rows per wavefront load (one row per CPR lanes)
  constexpr int NLD = kGqaTile / RPL;         // loads per tile, for K and for V
  constexpr int VT = kGqaTile * D;            // bf16 elements of one tile
  constexpr int SPP = kPage / TPW;            // partials per page
  constexpr int kWaves = kDecThreads / 64;
  __shared__ __attribute__((aligned(1024))) bf16 ktile[kWaves][VT];
  __shared__ __attribute__((aligned(1024))) bf16 vtile[kWaves][VT];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5, n = lane & 31;
  // Wavefront unit = (sequence, split, key/value head, head block), head block
  // fastest, then key/value head: the waves of a workgroup read neighbouring
  // rows of the same tokens.
  const int group = H / Hkv;
  const int nhb = (group + kGqaCols - 1) / kGqaCols;
  const int nsplit = max_blocks * SPP;
  long long unit = (long long)blockIdx.x * kWaves + wave;
  const int hb = (int)(unit % nhb);
  unit /= nhb;
  const int hkv = (int)(unit % Hkv);
  unit /= Hkv;
  const int sp = (int)(unit % nsplit);
  const int s = (int)(unit / nsplit);
  if (s >= S) return;  // padding of the last workgroup
  const int b = sp / SPP;                      // logical page
  const int t0 = (sp % SPP) * TPW;             // first slot of this split in the page
  // Both loads issue before the exit test (one memory latency, not two): the
  // empty asm consumes the table entry there, so it cannot sink below the test.
  const int len = seq_lens[s];
  const int entry = block_table[(size_t)s * max_blocks + b];
  asm volatile("" ::"s"(entry));
  const int ntok = min(TPW, len - b * kPage - t0);
  if (ntok <= 0) return;  // split past the sequence end
  const int page = min(max(entry, 0), num_pages - 1);
  const int cols = min(kGqaCols, group - hb * kGqaCols);  // query heads of this block
  const int hq0 = hkv * group + hb * kGqaCols;             // its first query head

  // K and V rows of this key/value head over the split's valid tokens only:
  // a token at or past ntok reads as zero and is never fetched.
  const uint32_t tok_bytes = (uint32_t)Hkv * D * 2;
  const bf16* kbase = pool + (size_t)page * 2 * kPage * Hkv * D + (size_t)t0 * Hkv * D + (size_t)hkv * D;
  const auto rk = make_rsrc(kbase, (uint32_t)ntok * tok_bytes);
  const auto rv = make_rsrc(kbase + (size_t)kPage * Hkv * D, (uint32_t)ntok * tok_bytes);
  bf16* kt = &ktile[wave][0];
  bf16* vt = &vtile[wave][0];
  // Tile loads read whole rows: CPR lanes cover one token's D features, so
  // each load instruction fetches RPL complete rows.
  const int ld_row = lane / CPR, ld_c = lane % CPR;
  const uint32_t ld_off = (uint32_t)ld_row * tok_bytes + 16u * ld_c;
  u32x4 kst[NLD], vst[NLD];
  auto load = [&](int t) {  // tile t into the staging registers (rows past ntok: zeros, no fetch)
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const uint32_t off = (uint32_t)(kGqaTile * t + RPL * i) * tok_bytes + ld_off;
      kst[i] = buf_load16_stream(rk, off);
      vst[i] = buf_load16_stream(rv, off);
    }
  };
  // Staging registers -> LDS: K row r, chunk c at c ^ k_swz(r) (read back as
  // operand rows), V at c ^ v_swz(r) (read back transposed).
  int kw_off[NLD], vw_off[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int row = RPL * i + ld_row;
    kw_off[i] = row * D + ((ld_c ^ k_swz<D>(row)) << 3);
    vw_off[i] = row * D + ((ld_c ^ v_swz<D>(row)) << 3);
  }
  load(0);  // first tile in flight before the query loads
  __builtin_amdgcn_sched_barrier(0);
  // Operand reads of Sᵀ = K·Qᵀ: lane n takes tile row perm_row(n), chunk 2kk + g.
  const int krow = perm_row(n);
  const int kr_base = krow * D, kr_swz = k_swz<D>(krow);

  // Qᵀ as the B operand: column n is query head hq0 + n (zero past the block's heads).
  bf16x8 qreg[KSTEPS];
  {
    const bf16* qrow = q + ((size_t)s * H + hq0 + min(n, cols - 1)) * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      const u32x4 z = {0u, 0u, 0u, 0u};
      const u32x4 x = *reinterpret_cast<const u32x4*>(qrow + 16 * kk);
      qreg[kk] = __builtin_bit_cast(bf16x8, n < cols ? x : z);
    }
  }
  // Transposed V reads: rows 8(G>>1) + j/4 (+16kk), column 32bb + 16(G&1) + 4(j%4).
  const int G = lane >> 4, j16 = lane & 15;
  int voff[DBLK];
#pragma unroll
  for (int bb = 0; bb < DBLK; ++bb) {
    const int row = 8 * (G >> 1) + (j16 >> 2);
    const int col = 32 * bb + 16 * (G & 1) + 4 * (j16 & 3);
    voff[bb] = row * D + (((col >> 3) ^ v_swz<D>(row)) << 3) + (col & 7);
  }

  f32x16 oacc[DBLK];
#pragma unroll
  for (int bb = 0; bb < DBLK; ++bb) oacc[bb] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;
  const int nt = (ntok + kGqaTile - 1) / kGqaTile;

  for (int t = 0; t < nt; ++t) {
    // Tile t lands; it moves to LDS and the staging registers take tile t+1
    // (past the last tile those loads fall outside the buffer: nothing is fetched).
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      *reinterpret_cast<u32x4*>(kt + kw_off[i]) = kst[i];
      *reinterpret_cast<u32x4*>(vt + vw_off[i]) = vst[i];
    }
    load(t + 1);
    // Sᵀ (32 tokens x 32 heads); tokens past ntok masked.
    f32x16 st = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(kt + kr_base + (((2 * kk + g) ^ kr_swz) << 3));
      st = mfma32(__builtin_bit_cast(bf16x8, a), qreg[kk], st);
    }
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const bool dead = kGqaTile * t + crow(0, r, g) >= ntok;
      st[r] = dead ? kNegInf : st[r];
      mx = fmaxf(mx, st[r]);
    }
    mx = xhalf_max(mx) * scale_log2;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleThreshold)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2_fast(m_run - m_new);  // 0 on the first tile
      l_run *= alpha;
#pragma unroll
      for (int bb = 0; bb < DBLK; ++bb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[bb][r] *= alpha;
      m_run = m_new;
    }
    bf16x8 pb[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = exp2_fast(__builtin_fmaf(st[8 * h + 2 * j], scale_log2, -m_run));
        const float p1 = exp2_fast(__builtin_fmaf(st[8 * h + 2 * j + 1], scale_log2, -m_run));
        w[j] = pack_bf16x2(p0, p1);
        l_run += p0 + p1;
      }
      pb[h] = __builtin_bit_cast(bf16x8, w);
    }
    // Oᵀ += Vᵀ Pᵀ (V rows past ntok were loaded as zeros)
#pragma unroll
    for (int bb = 0; bb < DBLK; ++bb)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x4 lo = lds_read_tr4(vt + voff[bb] + 16 * kk * D);
        const bf16x4 hi = lds_read_tr4(vt + voff[bb] + 16 * kk * D + 4 * D);
        oacc[bb] = mfma32(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pb[kk], oacc[bb]);
      }
  }

  // Partial of this split for the block's heads: unnormalised Oᵀ column, max, normaliser.
  const float l_tot = xhalf_sum(l_run);
  if (n >= cols) return;
  float* out = part + (((size_t)s * H + hq0 + n) * nsplit + sp) * (D + 2);
#pragma unroll
  for (int bb = 0; bb < DBLK; ++bb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float2 lo, hi;
      lo.x = oacc[bb][4 * i];
      lo.y = oacc[bb][4 * i + 1];
      hi.x = oacc[bb][4 * i + 2];
      hi.y = oacc[bb][4 * i + 3];
      *reinterpret_cast<float2*>(out + 32 * bb + 8 * i + 4 * g) = lo;
      *reinterpret_cast<float2*>(out + 32 * bb + 8 * i + 4 * g + 2) = hi;
    }
  if (g == 0) {
    out[D] = m_run;
    out[D + 1] = l_tot;
  }
}

// One wavefront per (sequence, head): merge the per-split partial states.
// Lane j holds split j's (m, l); the output features are split over lanes
// and the splits' rows are loaded in independent batches of 32, the first
// batch issued together with the (m, l) loads so that a merge of up to 32
// splits waits on memory once.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(const float* __restrict__ part,
                                                          const int32_t* __restrict__ seq_lens,
                                                          bf16* __restrict__ O, float* __restrict__ LSE, int H,
                                                          int max_blocks, int split) {
  constexpr int PER = D / 64;
  constexpr int BATCH = 32;
  const int sh = blockIdx.x;
  const int s = sh / H;
  const int lane = threadIdx.x;
  const int nsplit = max_blocks * (kPage / split);
  const int ns = min(max(seq_lens[s], 0), max_blocks * kPage) / split +
                 (min(max(seq_lens[s], 0), max_blocks * kPage) % split != 0);  // splits that hold tokens
  const float* p = part + (size_t)sh * nsplit * (D + 2);
  bf16* orow = O + (size_t)sh * D;
  if (ns == 0) {  // a sequence with no cached token: empty softmax, O = 0 and LSE = -inf
#pragma unroll
    for (int e = 0; e < PER; ++e) orow[lane * PER + e] = (bf16)0.f;
    if (LSE != nullptr && lane == 0) LSE[sh] = kNegInf;
    return;
  }
  float v[BATCH][PER];
  auto load_rows = [&](int j0) {  // this lane's features of splits j0 .. j0+BATCH-1 (clamped)
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const float* pj = p + (size_t)min(j0 + i, ns - 1) * (D + 2) + lane * PER;
#pragma unroll
      for (int e = 0; e < PER; ++e) v[i][e] = pj[e];
    }
  };
  // (m, l) of split `lane` (the first 64 splits), then the first rows.
  const float m0 = lane < ns ? p[(size_t)lane * (D + 2) + D] : kNegInf;
  const float l0 = lane < ns ? p[(size_t)lane * (D + 2) + D + 1] : 0.f;
  load_rows(0);
  float m = m0, o[PER], lsum = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
  for (int j0 = 64; j0 < ns; j0 += 64) {  // more than 64 splits
    const int j = j0 + lane;
    m = fmaxf(m, j < ns ? p[(size_t)j * (D + 2) + D] : kNegInf);
  }
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  for (int j0 = 0; j0 < ns; j0 += 64) {
    const int j = j0 + lane;
    const float mj = j0 == 0 ? m0 : (j < ns ? p[(size_t)j * (D + 2) + D] : kNegInf);
    const float lj = j0 == 0 ? l0 : (j < ns ? p[(size_t)j * (D + 2) + D + 1] : 0.f);
    const float w = j < ns ? exp2_fast(mj - m) : 0.f;
    lsum += w * lj;
    const int cnt = min(64, ns - j0);
    for (int i0 = 0; i0 < cnt; i0 += BATCH) {
      if (j0 + i0 > 0) load_rows(j0 + i0);
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        const float wi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), (i0 + i) & 63));
        const float wk = (i0 + i < cnt) ? wi : 0.f;  // split j0+i0+i's weight
#pragma unroll
        for (int e = 0; e < PER; ++e) o[e] += wk * v[i][e];
      }
    }
  }
  for (int off = 32; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off);
  const float inv = 1.f / lsum;
#pragma unroll
  for (int e = 0; e < PER; ++e) orow[lane * PER + e] = (bf16)(o[e] * inv);
  if (LSE != nullptr && lane == 0) LSE[sh] = (m + log2_fast(lsum)) * kLn2;
}

template <int D, int HG>
hipError_t launch(const DecodeArgs& a) {
  const int hgroups = a.H / HG;
  const dim3 grid1((unsigned)(a.S * a.max_blocks * kSplitsPerPage * hgroups)), block1(kDecThreads);
  hipLaunchKernelGGL((decode_split_kernel<D, HG>), grid1, block1, 0, a.stream, static_cast<const bf16*>(a.q),
                     static_cast<const bf16*>(a.kv_pool), a.block_table, a.seq_lens, a.part, a.H, a.num_pages,
                     a.max_blocks, a.scale * kLog2e);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(a.S * a.H), dim3(64), 0, a.stream, a.part, a.seq_lens,
                     static_cast<bf16*>(a.o), a.lse, a.H, a.max_blocks, kSplit);
  return hipGetLastError();
}

template <int D, int TPW>
hipError_t launch_gqa_split(const DecodeArgs& a, long long nhb) {
  const long long units = (long long)a.S * a.max_blocks * (kPage / TPW) * a.Hkv * nhb;
  const dim3 grid1((unsigned)((units + kDecThreads / 64 - 1) / (kDecThreads / 64))), block1(kDecThreads);
  hipLaunchKernelGGL((decode_gqa_split_kernel<D, TPW>), grid1, block1, 0, a.stream, static_cast<const bf16*>(a.q),
                     static_cast<const bf16*>(a.kv_pool), a.block_table, a.seq_lens, a.part, a.S, a.H, a.Hkv,
                     a.num_pages, a.max_blocks, a.scale * kLog2e);
  return hipGetLastError();
}

template <int D>
hipError_t launch_gqa(const DecodeArgs& a) {
  const long long nhb = (a.H / a.Hkv + kGqaCols - 1) / kGqaCols;
  // Page-sized splits when the table holds enough (page, key/value head) units.
  const int split = (long long)a.S * a.max_blocks * a.Hkv * nhb >= kGqaPageUnits ? kPage : kPage / 2;
  hipError_t e = split == kPage ? launch_gqa_split<D, kPage>(a, nhb) : launch_gqa_split<D, kPage / 2>(a, nhb);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(a.S * a.H), dim3(64), 0, a.stream, a.part, a.seq_lens,
                     static_cast<bf16*>(a.o), a.lse, a.H, a.max_blocks, split);
  return hipGetLastError();
}

}  // namespace

hipError_t static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {  // once per device, with that device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a) {
  if (a.Hkv != a.H) return a.d == 128 ? launch_gqa<128>(a) : launch_gqa<64>(a);
  if (a.d == 128) return (a.H % 8 == 0) ? launch<128, 8>(a) : launch<128, 1>(a);
  return (a.H % 8 == 0) ? launch<64, 8>(a) : launch<64, 1>(a);
}

}  // namespace fa
