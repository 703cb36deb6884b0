// fa_bwd.hip -- recompute backward of exact attention, for gfx950.
//
// Method (interview answer "flash attention呢", 标准答 part 2; study card
// airsota.com/?p=1562, section 四 ②): the backward keeps neither S nor P; it reloads
// Q, K, V tiles and recomputes the local scores, turning them into probabilities with
// the log-sum-exp saved by the forward, P = exp(S - LSE).  The gradient relations the
// self-test page ("二十四：Flash Attention自测题", section D) asks for are
//   dV = P^T dO,  dP = dO V^T,  D_i = rowsum(dO * O),  dS = P * (dP - D_i),
//   dQ = scale * dS K,  dK = scale * dS^T Q.
//
// gfx950 mapping (three kernels in stream order):
//  1. bwd_pre: D_i = rowsum(dO * O) in fp32 and clearing of the fp32 dQ accumulator;
//  2. bwd_main: one workgroup per 128-key tile of a KV head; each of its 4 waves keeps
//     K, V and its own 32 keys' dK, dV accumulators in registers for the whole
//     kernel, and walks the query tiles (64 rows) of every query head of the GQA
//     group that can see the tile (causal: from the diagonal down).  Per query tile:
//     S = Q K^T (recompute), P, dV += P^T dO, dP = dO V^T, dS, dK += dS^T Q on
//     32x32x16 bf16 MFMA, then dS goes through LDS so each wave forms dQ for a
//     32-wide slice of the head dimension over all 128 keys and adds it into the fp32
//     accumulator with atomics.  Q and dO are staged row-major and transposed (keys of
//     the contraction permuted to the MFMA register order), prefetched one tile ahead;
//  3. bwd_dq: dQ = scale * accumulator, rounded to bf16.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kBwdBC = 128;  // keys per workgroup
constexpr int kBwdBR = 64;   // query rows per step

__device__ __forceinline__ int perm16(int k) {
  return (k & ~15) | (((k >> 2) & 1) << 3) | (((k >> 3) & 1) << 2) | (k & 3);
}

template <int D>
struct BwdTile {
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int CPR = D / 8;
  static constexpr int RPT = kBwdBR * CPR / 256;  // staged rows per thread (4 or 2)
  static constexpr int R_LD = D + 8;              // row-major pitch (elements)
  static constexpr int T_LD = kBwdBR + 8;         // transposed pitch
  static constexpr int S_LD = kBwdBC + 8;         // dS pitch
  static constexpr int QS = 0;
  static constexpr int QT = QS + kBwdBR * R_LD;
  static constexpr int DOS = QT + D * T_LD;
  static constexpr int DOT = DOS + kBwdBR * R_LD;
  static constexpr int DSS = DOT + D * T_LD;
  static constexpr int END = DSS + kBwdBR * S_LD;  // bf16 elements
};

// D_i = sum_d dO_id O_id, and zero the dQ accumulator row.
template <int D>
__global__ void __launch_bounds__(256) bwd_pre_kernel(BwdParams p) {
  constexpr int TPR = D / 8;            // threads per row
  constexpr int RPB = 256 / TPR;        // rows per block
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / TPR;  // over B * Hq * Nq
  const int col = 8 * (tid % TPR);
  const int64_t nrows = (int64_t)p.B * p.Hq * p.Nq;
  float sum = 0.f;
  if (row < nrows) {
    const int i = (int)(row % p.Nq);
    const int64_t bh = row / p.Nq;
    const int hq = (int)(bh % p.Hq), b = (int)(bh / p.Hq);
    const u32x4_t o = *reinterpret_cast<const u32x4_t*>(p.o + b * p.os0 + hq * p.os1 + (int64_t)i * p.os2 + col);
    const u32x4_t g = *reinterpret_cast<const u32x4_t*>(p.dout + b * p.dos0 + hq * p.dos1 + (int64_t)i * p.dos2 + col);
#pragma unroll
    for (int w = 0; w < 4; ++w) sum += bf16_lo(o[w]) * bf16_lo(g[w]) + bf16_hi(o[w]) * bf16_hi(g[w]);
    float* acc = p.dq_acc + row * D + col;
    *reinterpret_cast<f32x4_t*>(acc) = f32x4_t{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4_t*>(acc + 4) = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off, TPR);
  if (row < nrows && tid % TPR == 0) p.delta[row] = sum;
}

template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
bwd_main_kernel(BwdParams p) {
  using T = BwdTile<D>;
  constexpr int BC = kBwdBC, BR = kBwdBR;
  __shared__ __attribute__((aligned(16))) uint16_t smem[T::END];
  __shared__ __attribute__((aligned(16))) float lse2_s[BR];
  __shared__ __attribute__((aligned(16))) float delta_s[BR];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  int t = xcd_contiguous(blockIdx.x, gridDim.x);
  const int kt = t % p.nkt;  // causal: low key tiles (most query tiles) first
  t /= p.nkt;
  const int hkv = t % p.Hkv;
  const int b = t / p.Hkv;

  int lk = p.Nk;
  if (p.kv_lens) {
    lk = p.kv_lens[b];
    lk = lk < 0 ? 0 : (lk > p.Nk ? p.Nk : lk);
  }
  const int diag = lk - p.Nq;
  const int k0 = kt * BC;
  const int kw = k0 + wave * 32 + l32;  // this lane's key (column of S, P, dP, dS)
  const u32x4_t zero4 = {0u, 0u, 0u, 0u};

  // ---- resident K, V fragments (B operands of S = Q K^T and dP = dO V^T)
  u32x4_t kf[T::KS], vf[T::KS];
  {
    const uint16_t* krow = p.k + b * p.ks0 + hkv * p.ks1 + (int64_t)kw * p.ks2 + 8 * hi;
    const uint16_t* vrow = p.v + b * p.vs0 + hkv * p.vs1 + (int64_t)kw * p.vs2 + 8 * hi;
#pragma unroll
    for (int s = 0; s < T::KS; ++s) {
      kf[s] = kw < lk ? *reinterpret_cast<const u32x4_t*>(krow + 16 * s) : zero4;
      vf[s] = kw < lk ? *reinterpret_cast<const u32x4_t*>(vrow + 16 * s) : zero4;
    }
  }
  // ---- K as the B operand of dQ = dS K for this wave's 32-wide slice of the head dim:
  //      column d = 32*wave + l32, k-step ks covers keys 16 ks + 8 hi + (0..7).
  u32x4_t ktf[BC / 16];
  {
    const int d = 32 * wave + l32;
    const uint16_t* kcol = p.k + b * p.ks0 + hkv * p.ks1 + d;
#pragma unroll
    for (int ks = 0; ks < BC / 16; ++ks) {
      uint32_t w4[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int ka = k0 + 16 * ks + 8 * hi + e;
        const uint32_t x0 = (ka < lk && d < D) ? kcol[(int64_t)ka * p.ks2] : 0u;
        const uint32_t x1 = (ka + 1 < lk && d < D) ? kcol[(int64_t)(ka + 1) * p.ks2] : 0u;
        w4[e >> 1] = x0 | (x1 << 16);
      }
      ktf[ks] = u32x4_t{w4[0], w4[1], w4[2], w4[3]};
    }
  }

  f32x16_t dk[T::DB], dv[T::DB];
#pragma unroll
  for (int d = 0; d < T::DB; ++d) dk[d] = dv[d] = f32x16_t{};

  const int nqt = (p.Nq + BR - 1) / BR;
  int qt0 = 0;
  if (p.causal) {
    const int first_q = k0 - diag;  // first query row that sees key k0
    qt0 = first_q <= 0 ? 0 : first_q / BR;
  }
  const int per_head = (k0 < lk) ? (nqt > qt0 ? nqt - qt0 : 0) : 0;
  const int iters = per_head * p.G;

  // staging: thread holds rows vr0 .. vr0+RPT-1, 8 dims at column vcol
  const int vcol = tid % T::CPR;
  const int vr0 = T::RPT * (tid / T::CPR);
  u32x4_t qreg[T::RPT], doreg[T::RPT];
  float lse_reg = INFINITY, delta_reg = 0.f;

  auto load_tile = [&](int it) {
    const int gi = it / per_head, qt = qt0 + it % per_head;
    const int hq = hkv * p.G + gi;
    const int q0 = qt * BR;
    const uint16_t* qb = p.q + b * p.qs0 + hq * p.qs1 + 8 * vcol;
    const uint16_t* db = p.dout + b * p.dos0 + hq * p.dos1 + 8 * vcol;
#pragma unroll
    for (int i = 0; i < T::RPT; ++i) {
      const int q = q0 + vr0 + i;
      qreg[i] = q < p.Nq ? *reinterpret_cast<const u32x4_t*>(qb + (int64_t)q * p.qs2) : zero4;
      doreg[i] = q < p.Nq ? *reinterpret_cast<const u32x4_t*>(db + (int64_t)q * p.dos2) : zero4;
    }
    if (tid < BR) {
      const int q = q0 + tid;
      const int64_t r = ((int64_t)b * p.Hq + hq) * p.Nq + q;
      lse_reg = q < p.Nq ? p.lse[r] * kLog2e : INFINITY;
      delta_reg = q < p.Nq ? p.delta[r] : 0.f;
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < T::RPT; ++i) {
      *reinterpret_cast<u32x4_t*>(smem + T::QS + (vr0 + i) * T::R_LD + 8 * vcol) = qreg[i];
      *reinterpret_cast<u32x4_t*>(smem + T::DOS + (vr0 + i) * T::R_LD + 8 * vcol) = doreg[i];
    }
    const int pos = perm16(vr0);
#pragma unroll
    for (int src = 0; src < 2; ++src) {
      const u32x4_t* r = src ? doreg : qreg;
      uint16_t* base = smem + (src ? T::DOT : T::QT);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint16_t* even = base + (8 * vcol + 2 * w) * T::T_LD + pos;
        uint16_t* odd = even + T::T_LD;
        if constexpr (T::RPT == 4) {
          const uint32_t x0 = r[0][w], x1 = r[1][w], x2 = r[2][w], x3 = r[3][w];
          *reinterpret_cast<u32x2_t*>(even) =
              u32x2_t{(x0 & 0xffffu) | (x1 << 16), (x2 & 0xffffu) | (x3 << 16)};
          *reinterpret_cast<u32x2_t*>(odd) =
              u32x2_t{(x0 >> 16) | (x1 & 0xffff0000u), (x2 >> 16) | (x3 & 0xffff0000u)};
        } else {
          const uint32_t x0 = r[0][w], x1 = r[1][w];
          *reinterpret_cast<uint32_t*>(even) = (x0 & 0xffffu) | (x1 << 16);
          *reinterpret_cast<uint32_t*>(odd) = (x0 >> 16) | (x1 & 0xffff0000u);
        }
      }
    }
    if (tid < BR) {
      lse2_s[tid] = lse_reg;
      delta_s[tid] = delta_reg;
    }
  };

  if (iters > 0) {
    load_tile(0);
    store_tile();
  }
  __syncthreads();

  const float c = p.scale_log2;
  for (int it = 0; it < iters; ++it) {
    const int gi = it / per_head, qt = qt0 + it % per_head;
    const int hq = hkv * p.G + gi;
    const int q0 = qt * BR;
    if (it + 1 < iters) load_tile(it + 1);

    // (1) S = Q K^T, rows = queries of block qb, column = this lane's key
    f32x16_t s[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      s[qb] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(smem + T::QS + (32 * qb + l32) * T::R_LD +
                                                            16 * ks + 8 * hi);
        s[qb] = mfma32(a, kf[ks], s[qb]);
      }
    }
    // (2) P = exp(S - LSE), zero where the pair does not exist
    const bool edge = (kw >= lk) || (q0 + BR > p.Nq) ||
                      (p.causal && k0 + BC - 1 > q0 + diag);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int ql = 32 * qb + 8 * rg + 4 * hi;
        const f32x4_t l4 = *reinterpret_cast<const f32x4_t*>(lse2_s + ql);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float pv = fast_exp2(fmaf(s[qb][4 * rg + e], c, -l4[e]));
          if (edge) {
            const int q = q0 + ql + e;
            const bool vis = kw < lk && q < p.Nq && (!p.causal || kw <= q + diag);
            pv = vis ? pv : 0.f;
          }
          s[qb][4 * rg + e] = pv;
        }
      }
    // P^T as the A operand (rows = keys, k-elements = queries in register order)
    u32x4_t pa[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int w = 0; w < 4; ++w)
          pa[qb][h2][w] = pack_bf16(s[qb][8 * h2 + 2 * w], s[qb][8 * h2 + 2 * w + 1]);

    // (3) dV += P^T dO
#pragma unroll
    for (int d = 0; d < T::DB; ++d)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const u32x4_t bo = *reinterpret_cast<const u32x4_t*>(
              smem + T::DOT + (32 * d + l32) * T::T_LD + 32 * qb + 16 * h2 + 8 * hi);
          dv[d] = mfma32(pa[qb][h2], bo, dv[d]);
        }

    // (4) dP = dO V^T
    f32x16_t dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      dp[qb] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(smem + T::DOS + (32 * qb + l32) * T::R_LD +
                                                            16 * ks + 8 * hi);
        dp[qb] = mfma32(a, vf[ks], dp[qb]);
      }
    }
    // (5) dS = P * (dP - D_i); keep it as the A operand and publish it in LDS
    u32x4_t da[2][2];
    uint16_t* dss = smem + T::DSS + wave * 32 + l32;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int ql = 32 * qb + 8 * rg + 4 * hi;
        const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(delta_s + ql);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float ds = s[qb][4 * rg + e] * (dp[qb][4 * rg + e] - d4[e]);
          dp[qb][4 * rg + e] = ds;
        }
      }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t pk = pack_bf16(dp[qb][8 * h2 + 2 * w], dp[qb][8 * h2 + 2 * w + 1]);
          da[qb][h2][w] = pk;
          const int r = 8 * h2 + 2 * w;  // register index of the low half
          const int ql = 32 * qb + 8 * (r >> 2) + 4 * hi + (r & 3);
          dss[ql * T::S_LD] = static_cast<uint16_t>(pk & 0xffffu);
          dss[(ql + 1) * T::S_LD] = static_cast<uint16_t>(pk >> 16);
        }

    // (6) dK += dS^T Q  (scale applied at the end)
#pragma unroll
    for (int d = 0; d < T::DB; ++d)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const u32x4_t bq = *reinterpret_cast<const u32x4_t*>(
              smem + T::QT + (32 * d + l32) * T::T_LD + 32 * qb + 16 * h2 + 8 * hi);
          dk[d] = mfma32(da[qb][h2], bq, dk[d]);
        }
    __syncthreads();  // dS tile complete

    // (7) dQ[:, 32*wave .. +32) += dS K over the workgroup's 128 keys
    if (32 * wave < D) {
      f32x16_t dq[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        dq[qb] = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < BC / 16; ++ks) {
          const u32x4_t a = *reinterpret_cast<const u32x4_t*>(smem + T::DSS + (32 * qb + l32) * T::S_LD +
                                                              16 * ks + 8 * hi);
          dq[qb] = mfma32(a, ktf[ks], dq[qb]);
        }
      }
      float* dqa = p.dq_acc + (((int64_t)b * p.Hq + hq) * p.Nq + q0) * D + 32 * wave + l32;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ql = 32 * qb + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (q0 + ql < p.Nq) unsafeAtomicAdd(dqa + (int64_t)ql * D, dq[qb][r]);
        }
    }
    __syncthreads();  // every read of this tile's LDS is done
    if (it + 1 < iters) store_tile();
    __syncthreads();
  }

  // ---- dK = scale * acc, dV = acc, rounded to bf16; rows >= Nk are not stored
  //      (rows in [Lk, Nk) hold zeros).  Layout: column d = 32*blk + l32, register r
  //      holds key 8*(r/4) + 4*hi + r%4 of this wave's 32 keys.
  uint16_t* dkb = p.dk + b * p.dks0 + hkv * p.dks1;
  uint16_t* dvb = p.dv + b * p.dvs0 + hkv * p.dvs1;
#pragma unroll
  for (int d = 0; d < T::DB; ++d)
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const int key0 = k0 + wave * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
      const int col = 32 * d + l32;
      const uint32_t kk = pack_bf16(dk[d][r] * p.scale, dk[d][r + 1] * p.scale);
      const uint32_t vv = pack_bf16(dv[d][r], dv[d][r + 1]);
      if (key0 < p.Nk) {
        dkb[(int64_t)key0 * p.dks2 + col] = static_cast<uint16_t>(kk & 0xffffu);
        dvb[(int64_t)key0 * p.dvs2 + col] = static_cast<uint16_t>(vv & 0xffffu);
      }
      if (key0 + 1 < p.Nk) {
        dkb[(int64_t)(key0 + 1) * p.dks2 + col] = static_cast<uint16_t>(kk >> 16);
        dvb[(int64_t)(key0 + 1) * p.dvs2 + col] = static_cast<uint16_t>(vv >> 16);
      }
    }
}

// dQ = scale * accumulator -> bf16, eight elements per thread.
template <int D>
__global__ void __launch_bounds__(256) bwd_dq_kernel(BwdParams p) {
  constexpr int TPR = D / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = idx / TPR;
  if (row >= (int64_t)p.B * p.Hq * p.Nq) return;
  const int col = 8 * (int)(idx % TPR);
  const int i = (int)(row % p.Nq);
  const int64_t bh = row / p.Nq;
  const int hq = (int)(bh % p.Hq), b = (int)(bh / p.Hq);
  const float* a = p.dq_acc + row * D + col;
  const f32x4_t x = *reinterpret_cast<const f32x4_t*>(a);
  const f32x4_t y = *reinterpret_cast<const f32x4_t*>(a + 4);
  const float sc = p.scale;
  *reinterpret_cast<u32x4_t*>(p.dq + b * p.dqs0 + hq * p.dqs1 + (int64_t)i * p.dqs2 + col) =
      u32x4_t{pack_bf16(x[0] * sc, x[1] * sc), pack_bf16(x[2] * sc, x[3] * sc),
              pack_bf16(y[0] * sc, y[1] * sc), pack_bf16(y[2] * sc, y[3] * sc)};
}

template <typename K>
hipError_t launch(K kernel, int64_t grid, int block, const BwdParams& p, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  BwdParams local = p;
  void* args[] = {&local};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3((unsigned)grid), dim3(block),
                         args, 0, stream);
}

template <int D>
hipError_t launch_all(BwdParams p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.B * p.Hq * p.Nq;
  constexpr int RPB = 256 / (D / 8);
  hipError_t e = launch(bwd_pre_kernel<D>, (rows + RPB - 1) / RPB, 256, p, stream);
  if (e != hipSuccess) return e;
  p.nkt = (p.Nk + kBwdBC - 1) / kBwdBC;
  e = launch(bwd_main_kernel<D>, (int64_t)p.nkt * p.Hkv * p.B, 256, p, stream);
  if (e != hipSuccess) return e;
  return launch(bwd_dq_kernel<D>, (rows * (D / 8) + 255) / 256, 256, p, stream);
}

}  // namespace

size_t bwd_workspace_bytes(int B, int Hq, int Nq, int D) {
  const size_t rows = (size_t)B * Hq * Nq;
  return ((rows * 4 + 255) & ~size_t(255)) + ((rows * D * 4 + 255) & ~size_t(255));
}

hipError_t launch_bwd(const BwdParams& p, int D, hipStream_t stream) {
  return D == 128 ? launch_all<128>(p, stream) : launch_all<64>(p, stream);
}

}  // namespace fa
