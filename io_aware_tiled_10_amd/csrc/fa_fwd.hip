// fa_fwd.hip -- tiled forward attention with an online softmax, for gfx950.
//
// Method (V2/V3 article, aiqz.cc, sections "IO瓶颈分析" and "V2算法优化"; study card
// airsota.com/?p=1562, sections 三 and 四 ①): for one tile of query rows, stream the
// key/value blocks once, keep the running row maximum m, the running exponent sum l
// and an unnormalised fp32 accumulator; when m grows, rescale l and the accumulator
// by exp(m_old - m_new); divide by l once after the last block.  The score and
// probability tiles never leave the chip.
//
// gfx950 mapping of the bf16 kernel (a redesign, not the pages' A100/H100 layout):
//  * one workgroup = 4 waves = 128 query rows; each wave owns 32 rows outright (the
//    article's "Warp级并行" principle: no reduction across waves);
//  * a K/V block is 64 keys; K is staged row-major and V transposed into LDS, double
//    buffered: the global loads of block j+1 are in flight while block j computes;
//  * the scores are computed transposed, S^T = K Q^T, on 32x32x16 bf16 MFMA, so each
//    lane holds one query's scores: the row max / sum are lane-local plus a single
//    exchange between the two wave halves;
//  * the probabilities stay in registers as the B operand of O^T += V^T P^T; V^T is
//    stored with its keys permuted to match the score register order, so no shuffle
//    is needed between the two products;
//  * exp is exp2 with scale*log2(e) folded into one fma per score;
//  * causal: blocks above the diagonal are never visited, the mask is applied only
//    on blocks that cross it, and the heaviest query tiles are launched first;
//  * workgroups are ordered so tiles that share a KV head run on the same XCD.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kFwdBR = 128;  // query rows per workgroup
constexpr int kFwdBC = 64;   // keys per block

template <int D>
struct FwdTile {
  static constexpr int KS = D / 16;            // k-steps of S^T = K Q^T
  static constexpr int DB = D / 32;            // 32-row blocks of O^T
  static constexpr int CPR = D / 8;            // 16-byte chunks per K/V row
  static constexpr int KCH = kFwdBC * CPR / 256;  // K chunks per thread
  static constexpr int KPT = KCH;              // V keys per thread (8 dims each)
  static constexpr int K_LD = D + 8;           // LDS row pitch of K (elements)
  static constexpr int V_LD = kFwdBC + 8;      // LDS row pitch of V^T (elements)
  static constexpr int STAGE = kFwdBC * K_LD + D * V_LD;
};

// Position of key k (0..15 within its group of 16) in the transposed V tile.  The
// MFMA result puts key 8a + 4h + b (a, h in {0,1}, b in 0..3) of a 16-key step in
// wave half h, element 4a + b; storing it at 8h + 4a + b lets each lane fetch its
// eight V^T elements with one 16-byte read.
__device__ __forceinline__ int vt_pos(int k) {
  return (k & ~15) | (((k >> 2) & 1) << 3) | (((k >> 3) & 1) << 2) | (k & 3);
}

// The running maximum used as the exponent reference is only moved when a block's
// maximum exceeds it by more than this many powers of two (per-wave decision).  Until
// then probabilities may exceed 1 by at most 2^kLazyRescale, which bf16 P and the fp32
// sums absorb; the final O = acc / l and LSE = m*scale + ln(l) use the same reference,
// so the result is unchanged while almost every accumulator rescale is skipped.
constexpr float kLazyRescale = 8.f;

template <int D, bool OUT_F32>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
fwd_bf16_kernel(FwdParams p) {
  using T = FwdTile<D>;
  constexpr int BR = kFwdBR, BC = kFwdBC;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * T::STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  // ---- which tile: XCD-contiguous, KV-head-major, heavy causal tiles first
  int t = xcd_contiguous(blockIdx.x, gridDim.x);
  const int gi = t % p.G;
  t /= p.G;
  const int rank = t % p.nqt;
  t /= p.nqt;
  const int hkv = t % p.Hkv;
  const int b = t / p.Hkv;
  const int qt = p.causal ? p.nqt - 1 - rank : rank;
  const int hq = hkv * p.G + gi;

  int lk = p.Nk;
  if (p.kv_lens) {
    lk = p.kv_lens[b];
    lk = lk < 0 ? 0 : (lk > p.Nk ? p.Nk : lk);
  }
  const int diag = lk - p.Nq;  // key j visible to query i iff j <= i + diag
  const int q_wg0 = qt * BR;
  int kend = lk;
  if (p.causal) {
    const int lim = q_wg0 + BR + diag;  // one past the last key the tile's last row sees
    kend = lim < kend ? lim : kend;
  }
  if (kend < 0) kend = 0;
  const int nblk = (kend + BC - 1) / BC;

  const int qi = q_wg0 + wave * 32 + l32;  // this lane's query row

  if (nblk == 0) {  // no visible key for any row of the tile: O = 0, LSE = -inf
    if (qi < p.Nq) {
      if constexpr (OUT_F32) {
        float* orow = static_cast<float*>(p.o) + b * p.os0 + hq * p.os1 + (int64_t)qi * p.os2;
        for (int d = 4 * hi; d < D; d += 8) *reinterpret_cast<f32x4_t*>(orow + d) = f32x4_t{};
      } else {
        uint16_t* orow = static_cast<uint16_t*>(p.o) + b * p.os0 + hq * p.os1 + (int64_t)qi * p.os2;
        for (int d = 4 * hi; d < D; d += 8) *reinterpret_cast<u32x2_t*>(orow + d) = u32x2_t{};
      }
      if (p.lse && hi == 0) p.lse[((int64_t)b * p.Hq + hq) * p.Nq + qi] = -INFINITY;
    }
    return;  // uniform over the workgroup
  }

  // ---- Q^T fragments (B operand), loaded once; rows past Nq read as zero
  u32x4_t qf[T::KS];
  {
    const int64_t qpitch = p.qs2 * 2;
    const uint16_t* qtile = p.q + b * p.qs0 + hq * p.qs1 + (int64_t)q_wg0 * p.qs2;
    const auto rq = make_rsrc(qtile, rows_span(min(BR, p.Nq - q_wg0), qpitch, D * 2));
    const uint32_t off = (uint32_t)((wave * 32 + l32) * qpitch) + 16 * hi;
#pragma unroll
    for (int s = 0; s < T::KS; ++s) qf[s] = buf_load16(rq, off + 32 * s);
  }

  const uint16_t* kbase = p.k + b * p.ks0 + hkv * p.ks1;
  const uint16_t* vbase = p.v + b * p.vs0 + hkv * p.vs1;
  const int64_t kpitch = p.ks2 * 2, vpitch = p.vs2 * 2;
  // K staging: chunk c = tid + 256 i -> (row c / CPR, column c % CPR), coalesced rows.
  // V staging: lanes sharing a column hold consecutive 4-key (2-key) groups, so the
  // transposed LDS writes of 16 lanes cover one V^T row without bank conflicts.
  constexpr int VG = BC / T::KPT;  // key groups per block
  const int vkg = tid % VG, vcol = tid / VG;
  const int vk0 = T::KPT * vkg;
  uint32_t koff[T::KCH];
#pragma unroll
  for (int i = 0; i < T::KCH; ++i) {
    const int c = tid + 256 * i;
    koff[i] = (uint32_t)((c / T::CPR) * kpitch) + 16 * (c % T::CPR);
  }
  const uint32_t voff = (uint32_t)(vk0 * vpitch) + 16 * vcol;

  u32x4_t kreg[T::KCH], vreg[T::KPT];

  auto load_block = [&](int blk) {
    const int key0 = blk * BC;
    const int rows = min(BC, lk - key0);
    const auto rk = make_rsrc(kbase + (int64_t)key0 * p.ks2, rows_span(rows, kpitch, D * 2));
    const auto rv = make_rsrc(vbase + (int64_t)key0 * p.vs2, rows_span(rows, vpitch, D * 2));
#pragma unroll
    for (int i = 0; i < T::KCH; ++i) kreg[i] = buf_load16(rk, koff[i]);
#pragma unroll
    for (int i = 0; i < T::KPT; ++i) vreg[i] = buf_load16(rv, voff + (uint32_t)(i * vpitch));
  };

  auto store_block = [&](int st) {
    uint16_t* Ks = smem + st * T::STAGE;
    uint16_t* Vs = Ks + BC * T::K_LD;
#pragma unroll
    for (int i = 0; i < T::KCH; ++i) {
      const int c = tid + 256 * i, row = c / T::CPR, col = c % T::CPR;
      *reinterpret_cast<u32x4_t*>(Ks + row * T::K_LD + 8 * col) = kreg[i];
    }
    const int pos = vt_pos(vk0);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint16_t* even = Vs + (8 * vcol + 2 * w) * T::V_LD + pos;
      uint16_t* odd = even + T::V_LD;
      if constexpr (T::KPT == 4) {
        const uint32_t x0 = vreg[0][w], x1 = vreg[1][w], x2 = vreg[2][w], x3 = vreg[3][w];
        *reinterpret_cast<u32x2_t*>(even) =
            u32x2_t{(x0 & 0xffffu) | (x1 << 16), (x2 & 0xffffu) | (x3 << 16)};
        *reinterpret_cast<u32x2_t*>(odd) =
            u32x2_t{(x0 >> 16) | (x1 & 0xffff0000u), (x2 >> 16) | (x3 & 0xffff0000u)};
      } else {
        const uint32_t x0 = vreg[0][w], x1 = vreg[1][w];
        *reinterpret_cast<uint32_t*>(even) = (x0 & 0xffffu) | (x1 << 16);
        *reinterpret_cast<uint32_t*>(odd) = (x0 >> 16) | (x1 & 0xffff0000u);
      }
    }
  };

  f32x16_t acc[T::DB];
#pragma unroll
  for (int d = 0; d < T::DB; ++d) acc[d] = f32x16_t{};
  float m = -INFINITY, l = 0.f;  // m: exponent reference (raw score units)
  const float c = p.scale_log2;
  const float thresh = kLazyRescale / c;

  load_block(0);
  store_block(0);
  __syncthreads();

  for (int j = 0; j < nblk; ++j) {
    const int st = j & 1;
    if (j + 1 < nblk) load_block(j + 1);
    const uint16_t* Ks = smem + st * T::STAGE;
    const uint16_t* Vs = Ks + BC * T::K_LD;

    // S^T = K Q^T for keys [0,32) and [32,64) of the block
    f32x16_t s0{}, s1{};
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) {
      const u32x4_t a0 = *reinterpret_cast<const u32x4_t*>(Ks + l32 * T::K_LD + 16 * ks + 8 * hi);
      const u32x4_t a1 =
          *reinterpret_cast<const u32x4_t*>(Ks + (32 + l32) * T::K_LD + 16 * ks + 8 * hi);
      s0 = mfma32(a0, qf[ks], s0);
      s1 = mfma32(a1, qf[ks], s1);
    }

    const int key0 = j * BC;
    const bool edge = (key0 + BC > lk) || (p.causal && key0 + BC - 1 > q_wg0 + diag);
    if (edge) {
      const int last = p.causal ? min(lk - 1, qi + diag) : lk - 1;  // last visible key
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (key > last) s0[r] = -INFINITY;
        if (key + 32 > last) s1[r] = -INFINITY;
      }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
    mx = halves_max(mx);
    // move the reference only when some row of the wave grew past the threshold
    if (__builtin_amdgcn_ballot_w64(mx > m + thresh || (m == -INFINITY && mx != -INFINITY))) {
      const float m_new = fmaxf(m, mx);
      const float alpha = m == -INFINITY ? 0.f : fast_exp2((m - m_new) * c);
      l *= alpha;
#pragma unroll
      for (int d = 0; d < T::DB; ++d) acc[d] *= alpha;
      m = m_new;
    }
    const float mc = (m == -INFINITY ? 0.f : m) * c;

    u32x4_t pf[4];
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = fast_exp2(fmaf(s0[r], c, -mc)), p1 = fast_exp2(fmaf(s0[r + 1], c, -mc));
      const float p2 = fast_exp2(fmaf(s1[r], c, -mc)), p3 = fast_exp2(fmaf(s1[r + 1], c, -mc));
      rs += (p0 + p1) + (p2 + p3);
      pf[r >> 3][(r & 7) >> 1] = pack_bf16(p0, p1);
      pf[2 + (r >> 3)][(r & 7) >> 1] = pack_bf16(p2, p3);
    }
    l += rs;

#pragma unroll
    for (int d = 0; d < T::DB; ++d) {
#pragma unroll
      for (int ts = 0; ts < 4; ++ts) {
        const u32x4_t a =
            *reinterpret_cast<const u32x4_t*>(Vs + (32 * d + l32) * T::V_LD + 16 * ts + 8 * hi);
        acc[d] = mfma32(a, pf[ts], acc[d]);
      }
    }

    if (j + 1 < nblk) store_block(st ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l once; LSE = m * scale + ln(l)
  const float lt = halves_sum(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (qi < p.Nq) {
    if constexpr (OUT_F32) {
      float* orow = static_cast<float*>(p.o) + b * p.os0 + hq * p.os1 + (int64_t)qi * p.os2;
#pragma unroll
      for (int d = 0; d < T::DB; ++d)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg)
          *reinterpret_cast<f32x4_t*>(orow + 32 * d + 8 * rg + 4 * hi) =
              f32x4_t{acc[d][4 * rg] * inv, acc[d][4 * rg + 1] * inv, acc[d][4 * rg + 2] * inv,
                      acc[d][4 * rg + 3] * inv};
    } else {
      uint16_t* orow = static_cast<uint16_t*>(p.o) + b * p.os0 + hq * p.os1 + (int64_t)qi * p.os2;
#pragma unroll
      for (int d = 0; d < T::DB; ++d)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg)
          *reinterpret_cast<u32x2_t*>(orow + 32 * d + 8 * rg + 4 * hi) =
              u32x2_t{pack_bf16(acc[d][4 * rg] * inv, acc[d][4 * rg + 1] * inv),
                      pack_bf16(acc[d][4 * rg + 2] * inv, acc[d][4 * rg + 3] * inv)};
    }
    if (p.lse && hi == 0)
      p.lse[((int64_t)b * p.Hq + hq) * p.Nq + qi] = lt > 0.f ? m * p.scale + __logf(lt) : -INFINITY;
  }
}

// fp32 inputs, D = 64: one lane per query row, K/V blocks of 32 keys broadcast from
// LDS, fp32 FMA on the vector units (the small fp32 workload is launch-bound; the
// matrix cores are reserved for the bf16 path).
constexpr int kF32BR = 64, kF32BC = 32;

template <int D>
__global__ void __launch_bounds__(64) fwd_f32_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(16))) float ks[kF32BC][D];
  __shared__ __attribute__((aligned(16))) float vs[kF32BC][D];
  const int tid = threadIdx.x;

  int t = xcd_contiguous(blockIdx.x, gridDim.x);
  const int gi = t % p.G;
  t /= p.G;
  const int rank = t % p.nqt;
  t /= p.nqt;
  const int hkv = t % p.Hkv;
  const int b = t / p.Hkv;
  const int qt = p.causal ? p.nqt - 1 - rank : rank;
  const int hq = hkv * p.G + gi;

  int lk = p.Nk;
  if (p.kv_lens) {
    lk = p.kv_lens[b];
    lk = lk < 0 ? 0 : (lk > p.Nk ? p.Nk : lk);
  }
  const int diag = lk - p.Nq;
  const int q_wg0 = qt * kF32BR;
  int kend = lk;
  if (p.causal) {
    const int lim = q_wg0 + kF32BR + diag;
    kend = lim < kend ? lim : kend;
  }
  if (kend < 0) kend = 0;
  const int qi = q_wg0 + tid;
  const int last = p.causal ? min(lk - 1, qi + diag) : lk - 1;

  const float* qsrc = static_cast<const float*>(static_cast<const void*>(p.q));
  const float* ksrc = static_cast<const float*>(static_cast<const void*>(p.k)) + b * p.ks0 + hkv * p.ks1;
  const float* vsrc = static_cast<const float*>(static_cast<const void*>(p.v)) + b * p.vs0 + hkv * p.vs1;

  float q[D], acc[D];
  const float c = p.scale_log2;
  const float* qrow = qsrc + b * p.qs0 + hq * p.qs1 + (int64_t)qi * p.qs2;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    q[d] = qi < p.Nq ? qrow[d] : 0.f;
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  for (int key0 = 0; key0 < kend; key0 += kF32BC) {
    __syncthreads();
    for (int e = tid; e < kF32BC * D / 4; e += 64) {
      const int row = e / (D / 4), col = 4 * (e % (D / 4));
      const int key = key0 + row;
      f32x4_t kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (key < lk) {
        kv = *reinterpret_cast<const f32x4_t*>(ksrc + (int64_t)key * p.ks2 + col);
        vv = *reinterpret_cast<const f32x4_t*>(vsrc + (int64_t)key * p.vs2 + col);
      }
      *reinterpret_cast<f32x4_t*>(&ks[row][col]) = kv;
      *reinterpret_cast<f32x4_t*>(&vs[row][col]) = vv;
    }
    __syncthreads();
    float s[kF32BC];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kF32BC; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) dot = fmaf(q[d], ks[j][d], dot);
      s[j] = key0 + j > last ? -INFINITY : dot;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2((m - m_use) * c);
    const float mc = m_use * c;
    l *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] *= alpha;
#pragma unroll
    for (int j = 0; j < kF32BC; ++j) {
      const float pj = fast_exp2(fmaf(s[j], c, -mc));
      l += pj;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(pj, vs[j][d], acc[d]);
    }
    m = m_new;
  }

  if (qi < p.Nq) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* orow = static_cast<float*>(p.o) + b * p.os0 + hq * p.os1 + (int64_t)qi * p.os2;
#pragma unroll
    for (int d = 0; d < D; d += 4)
      *reinterpret_cast<f32x4_t*>(orow + d) =
          f32x4_t{acc[d] * inv, acc[d + 1] * inv, acc[d + 2] * inv, acc[d + 3] * inv};
    if (p.lse) p.lse[((int64_t)b * p.Hq + hq) * p.Nq + qi] = l > 0.f ? m * p.scale + __logf(l) : -INFINITY;
  }
}

template <typename K>
hipError_t launch(K kernel, int grid, int block, const FwdParams& p, hipStream_t stream) {
  FwdParams local = p;
  void* args[] = {&local};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(grid), dim3(block), args, 0,
                         stream);
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p0, int in_dtype, int out_dtype, int D, hipStream_t stream) {
  FwdParams p = p0;
  if (in_dtype == FA_F32) {
    p.nqt = (p.Nq + kF32BR - 1) / kF32BR;
    const int64_t grid = (int64_t)p.nqt * p.Hq * p.B;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    return launch(fwd_f32_kernel<64>, (int)grid, 64, p, stream);
  }
  p.nqt = (p.Nq + kFwdBR - 1) / kFwdBR;
  const int64_t grid = (int64_t)p.nqt * p.Hq * p.B;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const bool of32 = out_dtype == FA_F32;
  if (D == 128)
    return of32 ? launch(fwd_bf16_kernel<128, true>, (int)grid, 256, p, stream)
                : launch(fwd_bf16_kernel<128, false>, (int)grid, 256, p, stream);
  return of32 ? launch(fwd_bf16_kernel<64, true>, (int)grid, 256, p, stream)
              : launch(fwd_bf16_kernel<64, false>, (int)grid, 256, p, stream);
}

}  // namespace fa
