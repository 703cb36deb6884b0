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
// gfx950 mapping (two kernels in stream order, no atomics: every output element is
// written once, so the backward is deterministic):
//  1. bwd_q: the forward's layout turned to dQ.  One workgroup (8 waves, 256 rows; with
//     dropout 4 waves, 128 rows) per query tile, Q and dO rows resident as MFMA operands,
//     K/V blocks of 64 keys through an LDS ring; per block S^T = K Q^T and dP^T = V dO^T
//     (one lane per query), P^T = exp(S^T - LSE), dS^T = P^T (dP^T - D_i), and
//     dQ^T += K^T dS^T with K^T from transposing reads; dQ = scale * acc, once.  Each
//     lane first forms its row's statistics, LSE * log2(e) and -D_i = -rowsum(dO * O)
//     in fp32, and stores them in two planes for the next kernel (the row's dO is
//     loaded anyway; every row of every query tile is covered, whether or not it sees
//     a key).  Recomputing S and dP here costs two more products per (query, key) pair
//     than accumulating dQ inside bwd_kv, but removes the device-scope fp32 atomics,
//     which on a multi-XCD part are executed beyond the per-XCD L2;
//  2. bwd_kv: one workgroup (8 waves) per 128-key tile of a KV head, walking the 64-row
//     query tiles of every query head of the GQA group that can see the tile (causal:
//     from the diagonal down).  Q, dO and the row statistics of each tile stream from
//     L2/HBM straight into a three-slot LDS ring (LDS DMA, XOR-swizzled 16-byte slots).
//     Each 32-key group is served by two waves: one keeps the keys' K rows and forms
//     S = Q K^T, P and dV += P^T dO; the other keeps their V rows and forms dP = dO V^T,
//     dS = P (dP - D_i) (P read from LDS) and dK += dS^T Q, one query tile behind the
//     first, so it never waits for P inside a step (with dropout both take the same
//     tile and meet at a barrier).  On
//     32x32x16 bf16 MFMA with one lane per key, P and dS are already the A operands of
//     the second products, whose dO^T and Q^T come from transposing LDS reads.
#include <type_traits>
#include <utility>

#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

// f(std::integral_constant<int, s>{}) for s = 0 .. N - 1, in order: a loop over ring
// slots whose index is a compile-time constant in each call.
template <typename F, int... S>
__device__ __forceinline__ void for_each_slot_impl(F&& f, std::integer_sequence<int, S...>) {
  (f(std::integral_constant<int, S>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void for_each_slot(F&& f) {
  for_each_slot_impl(f, std::make_integer_sequence<int, N>{});
}

// 16-byte slot swizzle of row r of a staged tile with `rowb`-byte rows: 16 consecutive
// rows read at one logical slot hit 16 different slots, and 8 consecutive rows read over
// an aligned group of 4 logical slots (transposing reads) cover every slot exactly twice.
template <int ROWB>
__host__ __device__ constexpr int swz_rows(int r) {
  constexpr int RPB = 256 / ROWB, SPR = ROWB / 16;
  const int a = r / RPB;
  return 4 * (a % (SPR / 4)) + (a / (SPR / 4)) % 4;
}
// The transposing reads address rows 16 ts + 8 r + v (v < 8) with the swizzle of row
// 8 r + v and step ts by an immediate: true when the swizzle repeats every 16 rows.
template <int ROWB>
constexpr bool swz_period_ok() {
  for (int r = 0; r < 64; ++r)
    if (swz_rows<ROWB>(r) != swz_rows<ROWB>(r % 16)) return false;
  return true;
}


// ------------------------------------------------------------------------------------
// dK/dV: key-tile outer loop, each 32-key group's work split between two waves.
// ------------------------------------------------------------------------------------
// Eight waves share a 128-key tile.  Waves 0-3 form S = Q K^T, P and dV += P^T dO for
// their 32 keys; waves 4-7 form dP = dO V^T, dS = P (dP - D_i) and dK += dS^T Q for the
// same keys, reading P from LDS.  Each wave keeps one operand (K or V) and one
// accumulator in registers, so two waves fit per SIMD and the two roles' MFMA and VALU
// phases interleave on it (one wave holding both, about 450 registers, ran one wave
// per SIMD with every LDS and MFMA latency exposed).  Without dropout, step s: the dV
// role takes tile s (S, P into one of two LDS buffers of its key group, dV) while the dK
// role takes tile s - 1 (dP, dS with the P the previous step's barrier published, dK);
// one barrier per step frees the ring slot and the P buffer.  With dropout both roles
// take tile s and a barrier in the middle publishes P and the mask table.
constexpr int kKvWaves = 8;
constexpr int kKvBC = 128;  // keys per workgroup (32 per key group)
constexpr int kKvBR = 64;   // query rows per tile
constexpr int kKvSlots = 3;  // ring depth

template <int D>
struct KvTile {
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int ROWB = D * 2;
  static constexpr int SPR = D / 8;
  static constexpr int RPI = 1024 / ROWB;
  static constexpr int QBYTES = kKvBR * ROWB;
  static constexpr int NDMA = QBYTES / (1024 * kKvWaves);            // per thread per tensor
  static constexpr int NDMA_KV = kKvBC * ROWB / (1024 * kKvWaves);
  static constexpr int STATS = 2 * QBYTES;
  static constexpr int SLOT = 2 * QBYTES + 1024;
  static constexpr int RING = kKvSlots * SLOT;
  // P of each key group: 32 fp32 per lane with dropout, else two 4 KiB bf16 buffers
  static constexpr int PX = RING;
  static constexpr int PXG = 32 * 64 * 4;           // bytes per key group
  static constexpr int KVBYTES = 2 * kKvBC * ROWB;  // K and V staging (set-up only)
  static constexpr int LDS_BYTES = PX + 4 * PXG > KVBYTES ? PX + 4 * PXG : KVBYTES;
  static_assert(NDMA * 1024 * kKvWaves == QBYTES, "a tile must split evenly over the waves");
  static_assert(NDMA_KV * 1024 * kKvWaves == kKvBC * ROWB, "K/V must split evenly");
  static __host__ __device__ constexpr int swz(int r) { return swz_rows<ROWB>(r); }
};

template <int D, bool DROP = false>
__global__ void __launch_bounds__(64 * kKvWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_kv_kernel(BwdParams p) {
  using T = KvTile<D>;
  constexpr int BC = kKvBC, BR = kKvBR, NW = kKvWaves, NS = kKvSlots;
  // dropout: per key group a 32 x 64 byte table of the tile's mask, [key][query]
  constexpr int ZBYTES = DROP ? 4 * 32 * BR : 0;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[T::LDS_BYTES + ZBYTES];
  unsigned char* ring = lds;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool dv_role = wave < 4;  // else the dP / dS / dK role
  const int kg = wave & 3;        // key group
  const int l32 = lane & 31, hi = lane >> 5;

  const TileId tix = tile_order(blockIdx.x, gridDim.x, p.B * p.Hkv, p.nkt, 1, true, p.gsz);
  const int kt = tix.rank;
  const int hkv = tix.pair % p.Hkv;
  const int b = tix.pair / p.Hkv;

  int lk = p.Nk;
  if (p.kv_lens) {
    lk = p.kv_lens[b];
    lk = lk < 0 ? 0 : (lk > p.Nk ? p.Nk : lk);
  }
  const int diag = lk - p.Nq;
  const int k0 = kt * BC;
  const int kwl = kg * 32 + l32;  // this lane's key within the tile (column of S, P, dS)
  const int kw = k0 + kwl;

  // DMA geometry: thread (wave w, lane) fills, for instruction i, row RPI (NW i + w) +
  // lane / SPR, slot lane % SPR
  const int drow = T::RPI * wave + lane / T::SPR, dslot = lane % T::SPR;
  const int dswz = dslot ^ T::swz(drow);
  auto dma_rows = [&](const uint16_t* base, int64_t pitch_el, int rows, int nrows_total,
                      unsigned char* dst, int ninst) {
    const int64_t pitch = pitch_el * 2;
    const auto rs = make_rsrc(base, rows_span(min(rows, nrows_total), pitch, D * 2));
    const uint32_t off = (uint32_t)(drow * pitch) + 16 * dswz;
    const int step = (int)(NW * T::RPI * pitch);
    for (int i = 0; i < ninst; ++i) lds_dma16(rs, dst + 1024 * (NW * i + wave), off, 0, step * i);
  };

  // ---- set-up: K and V tiles into LDS, then each wave's resident operand: K rows (dV
  //      role, B operand of S = Q K^T) or V rows (dK role, of dP = dO V^T)
  {
    const int valid = k0 < lk ? lk - k0 : 0;
    dma_rows(p.k + b * p.ks0 + hkv * p.ks1 + (int64_t)k0 * p.ks2, p.ks2, BC, valid, ring, T::NDMA_KV);
    dma_rows(p.v + b * p.vs0 + hkv * p.vs1 + (int64_t)k0 * p.vs2, p.vs2, BC, valid,
             ring + BC * T::ROWB, T::NDMA_KV);
    FA_WAIT_VMCNT(0);
    __syncthreads();
  }
  u32x4_t kv[T::KS];
  {
    const int sw = T::swz(kwl);
    const unsigned char* src = ring + (dv_role ? 0 : BC * T::ROWB);
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks)
      kv[ks] = *reinterpret_cast<const u32x4_t*>(src + kwl * T::ROWB + 16 * ((2 * ks + hi) ^ sw));
  }
  FA_WAIT_LGKMCNT0();
  __syncthreads();  // the ring reuses the staging area

  const int vg = lane >> 4, vi = lane & 15;
  const int vrow = 4 * (vg >> 1) + (vi >> 2);
  const int vlo = 2 * (vg & 1) + ((vi & 3) >> 1);

  f32x16_t acc[T::DB];  // dV (dV role) or dK / scale (dK role)
#pragma unroll
  for (int d = 0; d < T::DB; ++d) acc[d] = f32x16_t{};

  const int nqt = (p.Nq + BR - 1) / BR;
  int qt0 = 0;
  if (p.causal) {
    const int first_q = k0 - diag;
    qt0 = first_q <= 0 ? 0 : first_q / BR;
  }
  const int per_head = (k0 < lk) ? (nqt > qt0 ? nqt - qt0 : 0) : 0;
  const int iters = per_head * p.G;

  auto issue = [&](int it, int slot) {
    unsigned char* dst = ring + slot * T::SLOT;
    int gi = 0, q0 = 0, rows = 0;
    if (it < iters) {
      gi = it % p.G;
      q0 = (nqt - 1 - it / p.G) * BR;
      rows = p.Nq - q0;
    }
    const int hq = hkv * p.G + gi;
    if (wave < 2) {  // LSE * log2 e (wave 0) or -D_i (wave 1) of the tile's 64 rows
      const float* st = (wave == 0 ? p.lse2 : p.negd) + ((int64_t)b * p.Hq + hq) * p.Nq + q0;
      const auto rs = make_rsrc(st, rows <= 0 ? 0u : (uint32_t)(min(rows, BR) * 4));
      lds_dma4(rs, dst + T::STATS + 256 * wave, 4 * lane);
    }
    dma_rows(p.q + b * p.qs0 + hq * p.qs1 + (int64_t)q0 * p.qs2, p.qs2, BR, rows, dst, T::NDMA);
    dma_rows(p.dout + b * p.dos0 + hq * p.dos1 + (int64_t)q0 * p.dos2, p.dos2, BR, rows,
             dst + T::QBYTES, T::NDMA);
  };
  // the previous tile's loads must have landed: all but this wave's latest group (waves
  // 0 and 1 issue one statistics load more per tile)
  auto wait_ring = [&]() {
    if constexpr (T::NDMA == 2) {
      if (wave < 2) FA_WAIT_VMCNT(5); else FA_WAIT_VMCNT(4);
    } else {
      if (wave < 2) FA_WAIT_VMCNT(3); else FA_WAIT_VMCNT(2);
    }
  };
  static_assert(T::NDMA == 2 || T::NDMA == 1, "ring waits assume D = 128 or 64");

  const int qsw = T::swz(l32);
  const uint32_t ring_addr = lds_addr(ring);
  // transposing reads of slot 0 (dO for the dV role, Q for the dK role): rows 8 r + vrow
  // (+ 16 ts as an immediate), 32-column block blk
  uint32_t trb[2][T::DB];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int blk = 0; blk < T::DB; ++blk) {
      const int row = 8 * r + vrow;
      trb[r][blk] = ring_addr + (dv_role ? T::QBYTES : 0) + row * T::ROWB +
                    16 * ((4 * blk + vlo) ^ T::swz(row)) + 8 * (vi & 1);
    }
  static_assert(swz_period_ok<T::ROWB>(), "transposing-read swizzle must repeat every 16 rows");
  const float c = p.scale_log2;
  unsigned char* px = lds + T::PX + kg * T::PXG + 16 * lane;  // + 1024 per 4 registers
  unsigned char* zt = lds + T::LDS_BYTES + kg * 32 * BR;

  u32x4_t pkv[2][2];  // the dV role's P^T, kept from one step to the next without dropout

  // One query tile `it` in ring slot `slot` (uniform over the wave); `pboff` selects the
  // P buffer of the key group's pair.  `first`: the first product and the role's
  // elementwise work, leaving pk, the P^T (dV role) or dS^T (dK role) A operands of the
  // second product; `second`: the second product, from pk.
  auto tile = [&](int it, int slot, uint32_t pboff, bool first, bool second,
                  u32x4_t (&pk)[2][2]) __attribute__((always_inline)) {
    const int qt = nqt - 1 - it / p.G;
    const int q0 = qt * BR;
    const unsigned char* qs = ring + slot * T::SLOT;
    const float* stl = reinterpret_cast<const float*>(qs + T::STATS);        // LSE * log2 e
    const float* std_ = reinterpret_cast<const float*>(qs + T::STATS + 256);  // -D_i
    // 4 consecutive rows 32 qb + 8 rg + 4 hi .. of a statistics plane
    auto rows4 = [&](const float* plane, int qb, int rg) {
      return *reinterpret_cast<const f32x4_t*>(plane + 32 * qb + 8 * rg + 4 * hi);
    };

    // (1) S = Q K^T (dV role) or dP = dO V^T (dK role); rows = queries 32 qb + (register),
    //     column = key.  Without dropout the dK role starts its products from -D_i, so they
    //     leave dP - D_i, the factor of dS.
    if (first) {
    const unsigned char* arows = qs + (dv_role ? 0 : T::QBYTES);
    f32x16_t sp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      sp[qb] = f32x16_t{};
      if (!DROP && !dv_role) {
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const f32x4_t nd = rows4(std_, qb, rg);
#pragma unroll
          for (int e = 0; e < 4; ++e) sp[qb][4 * rg + e] = nd[e];
        }
      }
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) {
        const int o = (32 * qb + l32) * T::ROWB + 16 * ((2 * ks + hi) ^ qsw);
        sp[qb] = mfma32(*reinterpret_cast<const u32x4_t*>(arows + o), kv[ks], sp[qb]);
      }
    }

    // dropout: the mask of the group's 32 keys and the tile's 64 queries, drawn as the
    // forward draws it (lane L: the words of query q0 + L) and spread into the group's
    // [key][query] byte table; each role draws one of the two 16-key halves
    auto draw_mask_half = [&](int h2) {
      const int hq = hkv * p.G + (it % p.G);
      const u32x4_t w = dropout_words((k0 + 32 * kg) / 32, h2, q0 + lane, hq, b, p.seed_lo, p.seed_hi);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          zt[(4 * h2 + 8 * a + e) * BR + lane] = (unsigned char)((w[a] >> (8 * e)) & 0xffu);
    };
    // the table's 4-query word of this lane's key for query rows 32 qb + 8 rg + 4 hi ..
    auto mask_word = [&](int qb, int rg) {
      return *reinterpret_cast<const uint32_t*>(zt + l32 * BR + 32 * qb + 8 * rg + 4 * hi);
    };
    if (dv_role) {
      if constexpr (DROP) draw_mask_half(0);
      // P = exp(S - LSE), zero where the pair does not exist (two instances: tiles that
      // cross no edge test nothing); the plain P goes to the dK role through LDS, the
      // kept P / keep is the A operand of dV += P^T dO
      const bool edge = (k0 + BC > lk) || (q0 + BR > p.Nq) || (p.causal && k0 + BC - 1 > q0 + diag);
      auto probs = [&](auto masked) {
        constexpr bool M = decltype(masked)::value;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const int ql = 32 * qb + 8 * rg + 4 * hi;
            const f32x4_t l2 = rows4(stl, qb, rg);
            f32x4_t pv4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float pv = fast_exp2(fmaf(sp[qb][4 * rg + e], c, -l2[e]));
              if constexpr (M) {
                const int q = q0 + ql + e;
                const int lastk = min(lk - 1, p.causal ? q + diag : lk - 1);
                pv = ((q < p.Nq) & (kw <= lastk)) ? pv : 0.f;
              }
              pv4[e] = pv;
              sp[qb][4 * rg + e] = pv;
            }
            if constexpr (DROP) *reinterpret_cast<f32x4_t*>(px + 1024 * (4 * qb + rg)) = pv4;
          }
      };
      if (edge)
        probs(std::true_type{});
      else
        probs(std::false_type{});
      if constexpr (DROP) {  // dV takes the kept P / keep
        FA_WAIT_LGKMCNT0();  // P and this role's half of the mask table written
        FA_BARRIER();
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const uint32_t zw = mask_word(qb, rg);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              sp[qb][4 * rg + e] = dropout_keep(zw, e, p.drop_t) ? sp[qb][4 * rg + e] * p.drop_scale : 0.f;
          }
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int w = 0; w < 4; ++w)
            pk[qb][h2][w] = pack_bf16(sp[qb][8 * h2 + 2 * w], sp[qb][8 * h2 + 2 * w + 1]);
      if constexpr (!DROP) {  // without dropout the hand-off carries P as the bf16 dV uses
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2)
            *reinterpret_cast<u32x4_t*>(px + pboff + 1024 * (2 * qb + h2)) = pk[qb][h2];
      }
    } else {
      if constexpr (DROP) {
        draw_mask_half(1);
        FA_WAIT_LGKMCNT0();  // this role's half of the mask table written
        FA_BARRIER();        // P of this tile and the whole mask table published
      } else {
        asm volatile("" ::: "memory");  // the P reads below stay after the products above
      }
      // dS = P (dP - D_i) (with dropout: dP masked and scaled as the forward's P was)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          f32x4_t nd{};
          if constexpr (DROP) nd = rows4(std_, qb, rg);
          f32x4_t pv4;
          if constexpr (DROP) {
            pv4 = *reinterpret_cast<const f32x4_t*>(px + 1024 * (4 * qb + rg));
          } else {  // registers 4 rg .. 4 rg + 3: words 2 (rg % 2), +1 of pair (qb, rg / 2)
            const u32x2_t w2 =
                *reinterpret_cast<const u32x2_t*>(px + pboff + 1024 * (2 * qb + (rg >> 1)) + 8 * (rg & 1));
            pv4 = f32x4_t{bf16_lo(w2[0]), bf16_hi(w2[0]), bf16_lo(w2[1]), bf16_hi(w2[1])};
          }
          uint32_t zw = 0;
          if constexpr (DROP) zw = mask_word(qb, rg);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float dpz = sp[qb][4 * rg + e];  // dP - D_i, or dP with dropout
            if constexpr (DROP) dpz = (dropout_keep(zw, e, p.drop_t) ? dpz * p.drop_scale : 0.f) + nd[e];
            sp[qb][4 * rg + e] = pv4[e] * dpz;
          }
        }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int w = 0; w < 4; ++w)
            pk[qb][h2][w] = pack_bf16(sp[qb][8 * h2 + 2 * w], sp[qb][8 * h2 + 2 * w + 1]);
    }

    }  // first

    // (2) acc += pk x (dO rows for the dV role, Q rows for the dK role), k-step ts = 2 qb
    //     + h2 holding queries 16 ts + 8 (e/4) + 4 hi + e%4, which the transposing reads
    //     reproduce.  The 8 reads of 32-column block d + 1 are issued before the products
    //     of block d (LDS returns in order: with block d + 1's reads outstanding, a count
    //     of 8 means block d has arrived).
    if (second) {
      u32x2_t f[2][4][2];
      constexpr int TS = 16 * T::ROWB, SO = 0;
      const uint32_t soff = (uint32_t)__builtin_amdgcn_readfirstlane(slot * T::SLOT);
      auto tread = [&](int d, u32x2_t (&w)[4][2]) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const uint32_t a = trb[r][d] + soff;
          lds_read_tr16x2<SO, SO + TS>(w[0][r], w[1][r], a);
          lds_read_tr16x2<SO + 2 * TS, SO + 3 * TS>(w[2][r], w[3][r], a);
        }
      };
      tread(0, f[0]);
#pragma unroll
      for (int d = 0; d < T::DB; ++d) {
        u32x2_t (&w)[4][2] = f[d & 1];
        if (d + 1 < T::DB) {
          tread(d + 1, f[(d + 1) & 1]);
          lds_wait_tr<8>(w[0][0], w[0][1], w[1][0], w[1][1]);
          lds_wait_tr<8>(w[2][0], w[2][1], w[3][0], w[3][1]);
        } else {
          lds_wait_tr(w[0][0], w[0][1], w[1][0], w[1][1]);
          lds_wait_tr(w[2][0], w[2][1], w[3][0], w[3][1]);
        }
#pragma unroll
        for (int ts = 0; ts < 4; ++ts)
          acc[d] = mfma32(pk[ts >> 1][ts & 1],
                          u32x4_t{w[ts][0][0], w[ts][0][1], w[ts][1][0], w[ts][1][1]}, acc[d]);
      }
    }

  };
  // Without dropout the dK role runs one tile behind the dV role: in step s the dV role
  // forms P of tile s and the dK role uses P of tile s - 1, which the barrier closing step
  // s - 1 published (P alternates between two buffers per key group), so neither role
  // waits for the other inside a step.  The ring then loads one tile ahead: slots s - 1
  // (dK role), s (dV role) and s + 1 (loading) are in use, and iters + 1 steps run.  With
  // dropout both roles take tile s in step s (their barrier inside the tile publishes the
  // mask table) and the ring loads two tiles ahead.  Every wave passes the same barriers.
  // Without dropout the dV role also turns its work around: in step s it first adds
  // P(s - 1)^T dO(s - 1) (P kept in registers from step s - 1, dO still in slot s - 1), then
  // forms S and P of tile s.  Its exps then run beside the dK role's second product and
  // the dK role's dS work beside the dV role's products, instead of both roles' elementwise
  // work falling together between their products.
  constexpr int AHEAD = DROP ? 2 : 1, LAG = DROP ? 0 : 1;
  auto step = [&](int st, auto slot_c, auto role) __attribute__((always_inline)) {
    constexpr int slot = decltype(slot_c)::value;
    constexpr bool DV = decltype(role)::value;  // == dv_role
    issue(st + AHEAD, (slot + AHEAD) % NS);
    if (!DROP && DV) {
      if (st >= 1 && st - 1 < iters) tile(st - 1, (slot + NS - 1) % NS, 0u, false, true, pkv);
      if (st < iters) tile(st, slot, (uint32_t)(st & 1) * 4096u, true, false, pkv);
    } else {
      const int lag = DV ? 0 : LAG;
      const int it = st - lag;
      u32x4_t pk[2][2];
      if (it >= 0 && it < iters) tile(it, (slot + NS - lag) % NS, (uint32_t)(it & 1) * 4096u, true, true, pk);
    }
    if constexpr (DROP) wait_ring();  // tile st + 1 has landed (only st + 2 may be in flight)
    else FA_WAIT_VMCNT(0);            // tile st + 1 has landed
    FA_WAIT_LGKMCNT0();               // this wave's ring and P accesses are done
    FA_BARRIER();
  };
  static_assert(NS == 3, "the loop below walks three slots");
  if (iters > 0) {
    issue(0, 0);
    if constexpr (DROP) issue(1, 1);
    if constexpr (DROP) wait_ring();
    else FA_WAIT_VMCNT(0);
    FA_WAIT_LGKMCNT0();
    FA_BARRIER();
    const int nsteps = iters + LAG;
    // without dropout one loop per role (each with its own register allocation: the dV
    // role keeps its P from one step to the next); both pass the same barriers.  With
    // dropout the roles' steps do not depend on the role at compile time: one loop.
    auto run = [&](auto role) __attribute__((always_inline)) {
      int st = 0;
      for (; st + 2 < nsteps; st += 3) {
        step(st, std::integral_constant<int, 0>{}, role);
        step(st + 1, std::integral_constant<int, 1>{}, role);
        step(st + 2, std::integral_constant<int, 2>{}, role);
      }
      if (st < nsteps) step(st, std::integral_constant<int, 0>{}, role);
      if (st + 1 < nsteps) step(st + 1, std::integral_constant<int, 1>{}, role);
    };
    if (!DROP && dv_role)
      run(std::true_type{});
    else
      run(std::false_type{});
  }

  // ---- dV = acc (dV role) or dK = scale * acc (dK role), rounded to bf16; rows >= Nk
  //      are not stored.  Column d = 32 blk + l32, register r holds key 8 (r/4) + 4 hi +
  //      r%4 of the group's 32 keys.
  uint16_t* gb = dv_role ? p.dv + b * p.dvs0 + hkv * p.dvs1 : p.dk + b * p.dks0 + hkv * p.dks1;
  const int64_t gs = dv_role ? p.dvs2 : p.dks2;
  const float sc = dv_role ? 1.f : p.scale;
#pragma unroll
  for (int d = 0; d < T::DB; ++d)
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const int key0 = k0 + kg * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
      const int col = 32 * d + l32;
      const uint32_t g2 = pack_bf16(acc[d][r] * sc, acc[d][r + 1] * sc);
      if (key0 < p.Nk) gb[(int64_t)key0 * gs + col] = static_cast<uint16_t>(g2 & 0xffffu);
      if (key0 + 1 < p.Nk) gb[(int64_t)(key0 + 1) * gs + col] = static_cast<uint16_t>(g2 >> 16);
    }
}

// ------------------------------------------------------------------------------------
// dQ: query-tile outer loop, the forward's layout (one lane per query, K/V streamed).
// ------------------------------------------------------------------------------------
constexpr int kDqBC = 64;             // keys per block

template <int D, int NW, int NS, bool ROT = false>
struct DqTile {
  static constexpr int BR = 32 * NW;                         // query rows per workgroup
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int ROWB = D * 2;
  static constexpr int SPR = D / 8;
  static constexpr int RPI = 1024 / ROWB;
  static constexpr int TBYTES = kDqBC * ROWB;                // one K or V block
  static constexpr int NDMA = TBYTES / (1024 * NW);          // per thread per tensor
  // blocks in flight; with the rotated order a slot stays in use one block longer
  static constexpr int AHEAD = ROT ? NS - 2 : NS - 1;
  static_assert(AHEAD >= 1, "at least one block must be in flight");
  static constexpr int LDS_BYTES = 2 * NS * TBYTES;
  static_assert(NDMA * 1024 * NW == TBYTES, "a block must split evenly over the waves");
  static __device__ __forceinline__ int swz(int r) { return swz_rows<ROWB>(r); }
};

// NW waves (32 query rows each) per workgroup; NS-slot ring.  ROT: the second half of
// the waves takes each block's work in the rotated order (dQ of the previous block first,
// then S, dP and dS of this one), so the two waves of a SIMD run their elementwise work
// beside each other's products.
template <int D, int NW, int NS, bool DROP = false, bool ROT = false>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_q_kernel(BwdParams p) {
  using T = DqTile<D, NW, NS, ROT>;
  static_assert(!(ROT && DROP), "the rotated order is built for the path without dropout");
  constexpr int BR = T::BR, BC = kDqBC;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[T::LDS_BYTES];
  unsigned char* kring = lds;
  unsigned char* vring = lds + NS * T::TBYTES;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;

  // tile: ordered as the forward's (heavy causal tiles first inside each XCD's groups)
  const int nqt = (p.Nq + BR - 1) / BR;
  const TileId tix = tile_order(blockIdx.x, gridDim.x, p.B * p.Hkv, nqt, p.G, true, p.gsz);
  const int gi = tix.gi, rank = tix.rank;
  const int hkv = tix.pair % p.Hkv;
  const int b = tix.pair / p.Hkv;
  const int qt = p.causal ? nqt - 1 - rank : rank;
  const int hq = hkv * p.G + gi;

  int lk = p.Nk;
  if (p.kv_lens) {
    lk = p.kv_lens[b];
    lk = lk < 0 ? 0 : (lk > p.Nk ? p.Nk : lk);
  }
  const int diag = lk - p.Nq;
  const int q_wg0 = qt * BR;
  int kend = lk;
  if (p.causal) {
    const int lim = q_wg0 + BR + diag;
    kend = lim < kend ? lim : kend;
  }
  if (kend < 0) kend = 0;
  const int nblk = (kend + BC - 1) / BC;
  const int qi = q_wg0 + wave * 32 + l32;  // this lane's query row

  // Q and dO rows of this lane's query as B operands (k-elements = head dim); rows past
  // Nq read as zero.  The row's statistics: l2 = LSE log2 e (+inf for a row with no
  // visible key or past Nq, so its P is exactly zero) and D_i = sum_d dO_id O_id, from
  // the O row loaded in the same lane layout and the two halves' partial sums; both are
  // stored (as LSE log2 e and -D_i) for the dK/dV kernel, for every row below Nq,
  // including the rows of tiles that see no key.
  u32x4_t qf[T::KS], df[T::KS];
  float l2 = INFINITY, dd = 0.f;
  {
    const int rows = min(BR, p.Nq - q_wg0);
    const auto rq = make_rsrc(p.q + b * p.qs0 + hq * p.qs1 + (int64_t)q_wg0 * p.qs2,
                              rows_span(rows, p.qs2 * 2, D * 2));
    const auto rd = make_rsrc(p.dout + b * p.dos0 + hq * p.dos1 + (int64_t)q_wg0 * p.dos2,
                              rows_span(rows, p.dos2 * 2, D * 2));
    const auto ro = make_rsrc(p.o + b * p.os0 + hq * p.os1 + (int64_t)q_wg0 * p.os2,
                              rows_span(rows, p.os2 * 2, D * 2));
    const uint32_t oq = (uint32_t)((wave * 32 + l32) * p.qs2 * 2) + 16 * hi;
    const uint32_t od = (uint32_t)((wave * 32 + l32) * p.dos2 * 2) + 16 * hi;
    const uint32_t oo = (uint32_t)((wave * 32 + l32) * p.os2 * 2) + 16 * hi;
    float part = 0.f;
#pragma unroll
    for (int s = 0; s < T::KS; ++s) {
      df[s] = buf_load16(rd, od + 32 * s);
      const u32x4_t o = buf_load16(ro, oo + 32 * s);
#pragma unroll
      for (int w = 0; w < 4; ++w)
        part += bf16_lo(o[w]) * bf16_lo(df[s][w]) + bf16_hi(o[w]) * bf16_hi(df[s][w]);
    }
    dd = halves_sum(part);
    if (qi < p.Nq) {
      const int64_t row = ((int64_t)b * p.Hq + hq) * p.Nq + qi;
      const float L = p.lse[row];
      l2 = L == -INFINITY ? INFINITY : L * kLog2e;
      if (hi == 0) {
        p.lse2[row] = l2;
        p.negd[row] = -dd;
      }
    }
    if (nblk > 0) {
#pragma unroll
      for (int s = 0; s < T::KS; ++s) qf[s] = buf_load16(rq, oq + 32 * s);
    }
    asm volatile("" ::: "memory");  // issue these before the ring loads below
  }

  // (formed where it is used, so it is not held across the block loop)
  auto dq_row = [&]() { return p.dq + b * p.dqs0 + hq * p.dqs1 + (int64_t)qi * p.dqs2; };
  if (nblk == 0) {  // no visible key: dQ = 0
    if (qi < p.Nq) {
      uint16_t* dqrow = dq_row();
      for (int d = 4 * hi; d < D; d += 8) *reinterpret_cast<u32x2_t*>(dqrow + d) = u32x2_t{};
    }
    return;  // uniform over the workgroup
  }
  f32x16_t ndv;  // -D_i in every register: the start of each dP^T product without dropout
#pragma unroll
  for (int r = 0; r < 16; ++r) ndv[r] = -dd;

  const uint16_t* kbase = p.k + b * p.ks0 + hkv * p.ks1;
  const uint16_t* vbase = p.v + b * p.vs0 + hkv * p.vs1;
  const int64_t kpitch = p.ks2 * 2, vpitch = p.vs2 * 2;
  const int drow = T::RPI * wave + lane / T::SPR, dslot = lane % T::SPR;
  const int dswz = dslot ^ T::swz(drow);
  const uint32_t kdma = (uint32_t)(drow * kpitch) + 16 * dswz;
  const uint32_t vdma = (uint32_t)(drow * vpitch) + 16 * dswz;
  const int kstep = (int)(NW * T::RPI * kpitch), vstep = (int)(NW * T::RPI * vpitch);
  auto dma = [&](int blk, int slot) {  // blocks past the keys fill the slot with zeros
    const int key0 = blk * BC;
    const auto rk = make_rsrc(kbase + (int64_t)key0 * p.ks2, rows_span(min(BC, lk - key0), kpitch, D * 2));
    const auto rv = make_rsrc(vbase + (int64_t)key0 * p.vs2, rows_span(min(BC, lk - key0), vpitch, D * 2));
#pragma unroll
    for (int i = 0; i < T::NDMA; ++i)
      lds_dma16(rk, kring + slot * T::TBYTES + 1024 * (NW * i + wave), kdma, 0, kstep * i);
#pragma unroll
    for (int i = 0; i < T::NDMA; ++i)
      lds_dma16(rv, vring + slot * T::TBYTES + 1024 * (NW * i + wave), vdma, 0, vstep * i);
  };

  // transposing-read geometry for K^T (rows = keys 16 ts + 8 r + 4 (g/2) + i/4)
  const int vg = lane >> 4, vi = lane & 15;
  const int vrow = 4 * (vg >> 1) + (vi >> 2);
  const int vlo = 2 * (vg & 1) + ((vi & 3) >> 1);
  const int rsw = T::swz(l32);  // plain reads of key rows l32 and 32 + l32
  const uint32_t kring_addr = lds_addr(kring);

  f32x16_t acc[T::DB];
#pragma unroll
  for (int d = 0; d < T::DB; ++d) acc[d] = f32x16_t{};
  const float c = p.scale_log2;

  constexpr int kInFlight = 2 * T::NDMA * (T::AHEAD - 1);  // loads younger than block j+1
#pragma unroll
  for (int a = 0; a < T::AHEAD; ++a) dma(a, a);
  wait_vmcnt<kInFlight>();
  FA_BARRIER();

  // transposing reads of K in slot 0: rows 8 r + vrow (+ 16 ts and the slot offset as
  // immediates; the row swizzle repeats every 16 rows), 32-column block d
  static_assert(swz_period_ok<T::ROWB>(), "transposing-read swizzle must repeat every 16 rows");
  static_assert((NS - 1) * T::TBYTES + 3 * 16 * T::ROWB < 65536, "slot offsets must fit the immediate");
  uint32_t ktb[2][T::DB];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int d = 0; d < T::DB; ++d) {
      const int row = 8 * r + vrow;
      ktb[r][d] = kring_addr + row * T::ROWB + 16 * ((4 * d + vlo) ^ T::swz(row)) + 8 * (vi & 1);
    }

  // S, dP and dS of block j (slot `slot_c`, j % NS as a compile-time constant) into pf.
  auto sdp = [&](int j, auto slot_c, u32x4_t (&pf)[4]) __attribute__((always_inline)) {
    constexpr int slot = decltype(slot_c)::value;
    const unsigned char* ks = kring + slot * T::TBYTES;
    const unsigned char* vs = vring + slot * T::TBYTES;

    // Each 32-key half h of the block in turn: S^T = K Q^T and dP^T = V dO^T for keys
    // 32 h .. 32 h + 31 (without dropout dP^T starts from -D_i, so the products leave
    // dP^T - D_i), then P^T = exp(S^T - LSE) and dS^T = P^T (dP^T - D_i), zero where the
    // pair does not exist, packed as the B operand of dQ^T += K^T dS^T (k-step ts: keys
    // 16 ts + 8 (e/4) + 4 hi + e%4, e = 0..7).  The first half's elementwise work can run
    // beside the second half's products.
    const int key0 = j * BC;
    const bool edge = (key0 + BC > lk) || (p.causal && key0 + BC - 1 > q_wg0 + diag);
    const int last = p.causal ? min(lk - 1, qi + diag) : lk - 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x16_t sh{}, dph = DROP ? f32x16_t{} : ndv;
#pragma unroll
      for (int k = 0; k < T::KS; ++k) {
        const int o = (32 * h + l32) * T::ROWB + 16 * ((2 * k + hi) ^ rsw);
        const u32x4_t ak = *reinterpret_cast<const u32x4_t*>(ks + o);
        const u32x4_t av = *reinterpret_cast<const u32x4_t*>(vs + o);
        sh = mfma32(ak, qf[k], sh);
        dph = mfma32(av, df[k], dph);
      }
      // dropout: the forward's mask words of this lane's query for this half
      u32x4_t zw{};
      if constexpr (DROP) zw = dropout_words(key0 / 32 + h, hi, qi, hq, b, p.seed_lo, p.seed_hi);
      auto grads = [&](auto masked) {  // two instances: blocks crossing no edge test nothing
        constexpr bool M = decltype(masked)::value;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float v2[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const float pv = fast_exp2(fmaf(sh[r + e], c, -l2));
            float dpz = dph[r + e];  // dP - D_i, or dP with dropout
            if constexpr (DROP)
              dpz = (dropout_keep(zw[(r + e) >> 2], (r + e) & 3, p.drop_t) ? dpz * p.drop_scale : 0.f) - dd;
            float ds = pv * dpz;
            if constexpr (M) {
              const int key = key0 + 32 * h + 8 * ((r + e) >> 2) + 4 * hi + ((r + e) & 3);
              ds = key > last ? 0.f : ds;
            }
            v2[e] = ds;
          }
          pf[2 * h + (r >> 3)][(r & 7) >> 1] = pack_bf16(v2[0], v2[1]);
        }
      };
      if (edge)
        grads(std::true_type{});
      else
        grads(std::false_type{});
    }
  };

  // dQ^T += K^T dS^T for the block in slot `slot_c` with its dS^T in pf; K^T fragments
  // from transposing reads of the K block, those of 32-column block d + 1 issued before
  // the products of block d (LDS returns in order: with block d + 1's 8 reads
  // outstanding, a count of 8 means block d has arrived)
  auto dq = [&](auto slot_c, const u32x4_t (&pf)[4]) __attribute__((always_inline)) {
    constexpr int slot = decltype(slot_c)::value;
    {
      u32x2_t kt[2][4][2];
      constexpr int SO = slot * T::TBYTES, TS = 16 * T::ROWB;
      auto kread = [&](int d, u32x2_t (&w)[4][2]) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          lds_read_tr16x2<SO, SO + TS>(w[0][r], w[1][r], ktb[r][d]);
          lds_read_tr16x2<SO + 2 * TS, SO + 3 * TS>(w[2][r], w[3][r], ktb[r][d]);
        }
      };
      kread(0, kt[0]);
#pragma unroll
      for (int d = 0; d < T::DB; ++d) {
        u32x2_t (&w)[4][2] = kt[d & 1];
        if (d + 1 < T::DB) {
          kread(d + 1, kt[(d + 1) & 1]);
          lds_wait_tr<8>(w[0][0], w[0][1], w[1][0], w[1][1]);
          lds_wait_tr<8>(w[2][0], w[2][1], w[3][0], w[3][1]);
        } else {
          lds_wait_tr(w[0][0], w[0][1], w[1][0], w[1][1]);
          lds_wait_tr(w[2][0], w[2][1], w[3][0], w[3][1]);
        }
#pragma unroll
        for (int ts = 0; ts < 4; ++ts)
          acc[d] = mfma32(u32x4_t{w[ts][0][0], w[ts][0][1], w[ts][1][0], w[ts][1][1]}, pf[ts], acc[d]);
      }
    }

  };

  // One step j: load block j + AHEAD into the slot that is free, the block's work (the
  // rotated order first finishes block j - 1 with its dQ), then the barrier: block j + 1
  // has landed (only later blocks may be in flight), and the barrier publishes it and
  // frees the slot read longest ago.  Every wave passes the same barriers.
  auto run = [&](auto rot) __attribute__((always_inline)) {
    constexpr bool R = decltype(rot)::value;
    u32x4_t pf[4];
    auto step = [&](int j, auto slot_c) __attribute__((always_inline)) {
      constexpr int slot = decltype(slot_c)::value;
      dma(j + T::AHEAD, (slot + T::AHEAD) % NS);
      if constexpr (R) {
        if (j >= 1) dq(std::integral_constant<int, (slot + NS - 1) % NS>{}, pf);
        sdp(j, slot_c, pf);
      } else {
        sdp(j, slot_c, pf);
        dq(slot_c, pf);
      }
      wait_vmcnt<kInFlight>();
      FA_WAIT_LGKMCNT0();
      FA_BARRIER();
    };
    int j = 0;
    for (; j + NS - 1 < nblk; j += NS)
      for_each_slot<NS>([&](auto sc) { step(j + decltype(sc)::value, sc); });
    for_each_slot<NS - 1>([&](auto sc) {
      if (j + decltype(sc)::value < nblk) step(j + decltype(sc)::value, sc);
    });
    FA_WAIT_VMCNT(0);  // the trailing loads (past the keys: zeros) write the ring too
    if constexpr (R) {  // the last block's dQ, after the last barrier
      const int sl = (nblk - 1) % NS;
      for_each_slot<NS>([&](auto sc) {
        if (sl == decltype(sc)::value) dq(sc, pf);
      });
    }
  };
  if (ROT && wave >= NW / 2)
    run(std::bool_constant<ROT>{});
  else
    run(std::false_type{});

  // ---- dQ = scale * acc (lane = query row, register = head-dim element)
  if (qi < p.Nq) {
    const float sc = p.scale;
    uint16_t* dqrow = dq_row();
#pragma unroll
    for (int d = 0; d < T::DB; ++d)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg)
        *reinterpret_cast<u32x2_t*>(dqrow + 32 * d + 8 * rg + 4 * hi) =
            u32x2_t{pack_bf16(acc[d][4 * rg] * sc, acc[d][4 * rg + 1] * sc),
                    pack_bf16(acc[d][4 * rg + 2] * sc, acc[d][4 * rg + 3] * sc)};
  }
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

template <int D, bool DROP>
hipError_t launch_all(BwdParams p, hipStream_t stream) {
  // dQ first: it also writes the row statistics the dK/dV kernel reads.  Without dropout:
  // 256-row query tiles of 8 waves, the second four in the rotated order, on a four-slot
  // ring (two blocks ahead); with dropout: 128-row tiles of 4 waves, two workgroups per
  // compute unit, on a two-slot ring.
  // Each kernel's XCDs take the (batch entry, KV head) groups a few at a time, so that the
  // tiles in flight on an XCD share few groups' tensors in its L2: one group at a time
  // when every tile does the same work (non-causal), else enough groups for four tiles
  // per workgroup slot of the XCD's 32 compute units, so the longest-first order inside
  // each batch of groups still balances (with two tiles per slot the B2 H16 N4096 causal
  // backward ran 2-3 % slower).
  auto group_size = [&](int64_t tiles_per_group, int slots_per_cu) {
    if (!p.causal) return 1;
    const int64_t want = 4 * 32 * slots_per_cu;
    return (int)((want + tiles_per_group - 1) / tiles_per_group);
  };
  hipError_t e;
  if constexpr (DROP) {
    constexpr int NW = 4, NS = 2;
    const int64_t nqt = (p.Nq + 32 * NW - 1) / (32 * NW);
    p.gsz = group_size(nqt * p.G, 2);
    e = launch(bwd_q_kernel<D, NW, NS, true>, nqt * p.Hq * p.B, 64 * NW, p, stream);
  } else {
    constexpr int NW = 8, NS = 4;
    const int64_t nqt = (p.Nq + 32 * NW - 1) / (32 * NW);
    p.gsz = group_size(nqt * p.G, 1);
    e = launch(bwd_q_kernel<D, NW, NS, false, true>, nqt * p.Hq * p.B, 64 * NW, p, stream);
  }
  if (e != hipSuccess) return e;
  p.nkt = (p.Nk + kKvBC - 1) / kKvBC;
  p.gsz = group_size(p.nkt, 1);
  return launch(bwd_kv_kernel<D, DROP>, (int64_t)p.nkt * p.Hkv * p.B, 64 * kKvWaves, p, stream);
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p, int D, hipStream_t stream) {
  if (p.drop_t > 0)
    return D == 128 ? launch_all<128, true>(p, stream) : launch_all<64, true>(p, stream);
  return D == 128 ? launch_all<128, false>(p, stream) : launch_all<64, false>(p, stream);
}

}  // namespace fa
