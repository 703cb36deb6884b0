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
//  1. bwd_pre: per query row, D_i = rowsum(dO * O) in fp32 and LSE * log2(e), stored
//     side by side; the fp32 dQ accumulator row is cleared;
//  2. bwd_main: one workgroup (4 waves) per 128-key tile of a KV head.  Each wave keeps
//     its 32 keys' K and V rows (operands of S and dP), a 32-column slice of K^T (the
//     operand of dQ) and the fp32 dK, dV accumulators in registers, and walks the
//     64-row query tiles of every query head of the GQA group that can see the tile
//     (causal: from the diagonal down).  Q, dO and the row statistics of each tile
//     stream from L2/HBM straight into a three-slot LDS ring (LDS DMA, XOR-swizzled
//     16-byte slots), two tiles ahead.  Per tile: S = Q K^T and dP = dO V^T on
//     32x32x16 bf16 MFMA (one lane per key, so P and dS are already the A operands
//     of dV += P^T dO and dK += dS^T Q), with dO^T and Q^T from transposing LDS
//     reads; dS^T goes to LDS with 8-byte writes, and after one barrier each wave
//     reads dS back transposed to form its slice of dQ over the 128 keys, added into
//     the fp32 accumulator with atomics;
//  3. bwd_dq: dQ = scale * accumulator, rounded to bf16.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdBC = 32 * kBwdWaves;  // keys per workgroup (32 per wave)
constexpr int kBwdBR = 64;              // query rows per tile
constexpr int kBwdSlots = 3;            // ring depth: Q, dO and statistics of one tile

template <int D>
struct BwdTile {
  static constexpr int KS = D / 16;                       // k-steps over the head dim
  static constexpr int DB = D / 32;                       // 32-column blocks of the head dim
  static constexpr int ROWB = D * 2;                      // bytes per staged row
  static constexpr int SPR = D / 8;                       // 16-byte slots per row
  static constexpr int RPB = 256 / ROWB;                  // rows per 256-byte bank period
  static constexpr int RPI = 1024 / ROWB;                 // rows per wave DMA instruction
  static constexpr int QBYTES = kBwdBR * ROWB;            // one Q or dO tile
  static constexpr int NDMA = QBYTES / (1024 * kBwdWaves);  // per thread per tensor
  static constexpr int NDMA_KV = kBwdBC * ROWB / (1024 * kBwdWaves);
  static constexpr int STATS = 2 * QBYTES;                // offset of the statistics
  static constexpr int SLOT = 2 * QBYTES + 1024;          // Q, dO, 64 x (lse2, D_i) + pad
  static constexpr int RING = kBwdSlots * SLOT;
  static constexpr int KVBYTES = 2 * kBwdBC * ROWB;       // K and V tiles (set-up only)
  static constexpr int DS_ROWB = kBwdBR * 2;              // dS^T row: 64 queries, bf16
  static constexpr int DSBYTES = kBwdBC * DS_ROWB;        // one dS^T buffer
  static constexpr int DSOFF = RING > KVBYTES ? RING : KVBYTES;
  static constexpr int LDS_BYTES = DSOFF + 2 * DSBYTES;
  static constexpr int NSL = DB;                          // 32-wide dQ column slices
  static constexpr int QBW = 2 * NSL / kBwdWaves;         // 32-row dQ blocks per wave
  static_assert(NDMA * 1024 * kBwdWaves == QBYTES, "a tile must split evenly over the waves");
  // 16-byte slot swizzle of staged row r: 16 consecutive rows read at one logical slot
  // hit 16 different slots, and 8 consecutive rows read over an aligned group of 4
  // logical slots (transposing reads) cover every slot exactly twice
  static __device__ __forceinline__ int swz(int r) {
    const int a = r / RPB;
    return 4 * (a % (SPR / 4)) + (a / (SPR / 4)) % 4;
  }
};
// dS^T rows are 128 bytes: the geometry of a D = 64 tile
__device__ __forceinline__ int swz_ds(int r) { return BwdTile<64>::swz(r); }

// Per query row: stats = (LSE * log2 e, D_i = sum_d dO_id O_id); zero the dQ accumulator
// row.  Rows whose LSE is -inf (no visible key) get +inf, so their P is exactly zero.
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
  if (row < nrows && tid % TPR == 0) {
    const float L = p.lse[row];
    const float l2 = L == -INFINITY ? INFINITY : L * kLog2e;
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    reinterpret_cast<f32x2_t*>(p.stats)[row] = f32x2_t{l2, sum};
  }
}

template <int D>
__global__ void __launch_bounds__(64 * kBwdWaves) __attribute__((amdgpu_waves_per_eu(1, 1)))
bwd_main_kernel(BwdParams p) {
  using T = BwdTile<D>;
  constexpr int BC = kBwdBC, BR = kBwdBR, NW = kBwdWaves, NS = kBwdSlots;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[T::LDS_BYTES];
  unsigned char* ring = lds;
  unsigned char* dsbuf = lds + T::DSOFF;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int kwl = wave * 32 + l32;  // this lane's key within the tile (column of S, P, dS)
  const int kw = k0 + kwl;

  // DMA geometry shared by every staged tile: thread (wave w, lane) fills, for
  // instruction i, row RPI (NW i + w) + lane / SPR, slot lane % SPR; the row's swizzle
  // does not depend on i, whose row step goes into the scalar offset.
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

  // ---- set-up: K and V tiles into LDS, then the resident operands
  const uint16_t* kbase = p.k + b * p.ks0 + hkv * p.ks1 + (int64_t)k0 * p.ks2;
  const uint16_t* vbase = p.v + b * p.vs0 + hkv * p.vs1 + (int64_t)k0 * p.vs2;
  {
    const int valid = k0 < lk ? lk - k0 : 0;
    dma_rows(kbase, p.ks2, BC, valid, ring, T::NDMA_KV);
    dma_rows(vbase, p.vs2, BC, valid, ring + BC * T::ROWB, T::NDMA_KV);
    FA_WAIT_VMCNT(0);
    __syncthreads();
  }
  // K, V rows of this lane's key: B operands of S = Q K^T and dP = dO V^T
  u32x4_t kf[T::KS], vf[T::KS];
  {
    const int sw = T::swz(kwl);
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) {
      const int o = kwl * T::ROWB + 16 * ((2 * ks + hi) ^ sw);
      kf[ks] = *reinterpret_cast<const u32x4_t*>(ring + o);
      vf[ks] = *reinterpret_cast<const u32x4_t*>(ring + BC * T::ROWB + o);
    }
  }
  // Transposing-read geometry (lane 16 g + i reads row 16 ts + 8 r + 4 (g/2) + i/4 and 4
  // columns from 32 blk + 16 (g%2) + 4 (i%4)).  For any tile row period the swizzle of
  // that row is 4 X + (2 r + g/2) % 4 with X depending on the lane only.
  const int vg = lane >> 4, vi = lane & 15;
  const int vrow = 4 * (vg >> 1) + (vi >> 2);
  const int vlo = 2 * (vg & 1) + ((vi & 3) >> 1);
  auto tr_off = [&](int rowb, int r, int blk, int swz_row) {  // byte offset in a tile
    const int row = 8 * r + vrow;
    return row * rowb + 16 * ((4 * blk + vlo) ^ swz_row) + 8 * (vi & 1);
  };
  // K^T slice of this wave's dQ columns: B operand of dQ = dS K, keys in the order the
  // transposing reads of dS^T produce
  constexpr int QBW = T::QBW;                 // dQ row blocks of this wave
  const int dsl = wave % T::NSL;              // its 32-column slice of the head dim
  const int qb0 = (wave / T::NSL) * QBW;      // its first 32-row dQ block
  u32x4_t ktf[BC / 16];
#pragma unroll
  for (int ks = 0; ks < BC / 16; ++ks) {
    u32x2_t lo, up;
    const int r0 = 16 * ks + vrow, r1 = 16 * ks + 8 + vrow;
    const uint32_t a = lds_addr(ring);
    const uint32_t o0 = a + 16 * ks * T::ROWB + tr_off(T::ROWB, 0, dsl, T::swz(r0));
    const uint32_t o1 = a + 16 * ks * T::ROWB + tr_off(T::ROWB, 1, dsl, T::swz(r1));
    lds_read_tr16<0>(lo, o0);
    lds_read_tr16<0>(up, o1);
    lds_wait_tr2(lo, up);
    ktf[ks] = u32x4_t{lo[0], lo[1], up[0], up[1]};
  }
  FA_WAIT_LGKMCNT0();
  __syncthreads();  // the ring reuses the K/V staging area

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
  // Tile order: last query tile first, the group's heads innermost.  Every key tile of
  // a KV head then visits the same (query tile, head) at about the same time, so Q, dO
  // and the dQ accumulator rows of that tile are shared in L2 instead of being fetched
  // once per key tile.

  // one query tile `it` (head gi, tile qt) into ring slot `slot`; past the last tile
  // the descriptors are empty and the slot is filled with zeros
  auto issue = [&](int it, int slot) {
    unsigned char* dst = ring + slot * T::SLOT;
    int gi = 0, q0 = 0, rows = 0;
    if (it < iters) {
      gi = it % p.G;
      q0 = (nqt - 1 - it / p.G) * BR;
      rows = p.Nq - q0;
    }
    const int hq = hkv * p.G + gi;
    if (wave == 0) {  // (lse2, D_i) of the tile's 64 rows, 512 bytes
      const float* st = p.stats + 2 * (((int64_t)b * p.Hq + hq) * p.Nq + q0);
      const auto rs = make_rsrc(st, rows <= 0 ? 0u : (uint32_t)(min(rows, BR) * 8));
      lds_dma16(rs, dst + T::STATS, 16 * lane);
    }
    dma_rows(p.q + b * p.qs0 + hq * p.qs1 + (int64_t)q0 * p.qs2, p.qs2, BR, rows, dst, T::NDMA);
    dma_rows(p.dout + b * p.dos0 + hq * p.dos1 + (int64_t)q0 * p.dos2, p.dos2, BR, rows,
             dst + T::QBYTES, T::NDMA);
  };
  // the previous tile's loads must have landed: all but this wave's latest group
  auto wait_ring = [&]() {
    if constexpr (T::NDMA == 4) {
      if (wave == 0) FA_WAIT_VMCNT(9); else FA_WAIT_VMCNT(8);
    } else {
      if (wave == 0) FA_WAIT_VMCNT(5); else FA_WAIT_VMCNT(4);
    }
  };
  static_assert(T::NDMA == 4 || T::NDMA == 2, "ring waits assume D = 128 or 64");

  const int qsw = T::swz(l32);  // plain reads of query rows 32 qb + l32
  const uint32_t ring_addr = lds_addr(ring), ds_addr = lds_addr(dsbuf);
  const float c = p.scale_log2;

  if (iters > 0) {
    issue(0, 0);
    issue(1, 1);
    wait_ring();
    FA_BARRIER();
  }

  for (int it = 0; it < iters; ++it) {
    const int slot = it % NS;
    issue(it + 2, (it + 2) % NS);
    const int gi = it % p.G, qt = nqt - 1 - it / p.G;
    const int hq = hkv * p.G + gi;
    const int q0 = qt * BR;
    const unsigned char* qs = ring + slot * T::SLOT;
    const unsigned char* dos = qs + T::QBYTES;
    const float* st = reinterpret_cast<const float*>(qs + T::STATS);

    // (1) S = Q K^T and dP = dO V^T; rows = queries 32 qb + (register), column = key
    f32x16_t s[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      s[qb] = dp[qb] = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < T::KS; ++ks) {
        const int o = (32 * qb + l32) * T::ROWB + 16 * ((2 * ks + hi) ^ qsw);
        const u32x4_t aq = *reinterpret_cast<const u32x4_t*>(qs + o);
        const u32x4_t ad = *reinterpret_cast<const u32x4_t*>(dos + o);
        s[qb] = mfma32(aq, kf[ks], s[qb]);
        dp[qb] = mfma32(ad, vf[ks], dp[qb]);
      }
    }

    // (2) P = exp(S - LSE), dS = P (dP - D_i); zero where the pair does not exist
    const bool edge = (k0 + BC > lk) || (q0 + BR > p.Nq) || (p.causal && k0 + BC - 1 > q0 + diag);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int ql = 32 * qb + 8 * rg + 4 * hi;
        const f32x4_t st01 = *reinterpret_cast<const f32x4_t*>(st + 2 * ql);
        const f32x4_t st23 = *reinterpret_cast<const f32x4_t*>(st + 2 * ql + 4);
        const float l2[4] = {st01[0], st01[2], st23[0], st23[2]};
        const float dd[4] = {st01[1], st01[3], st23[1], st23[3]};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float pv = fast_exp2(fmaf(s[qb][4 * rg + e], c, -l2[e]));
          if (edge) {
            const int q = q0 + ql + e;
            const bool vis = kw < lk && q < p.Nq && (!p.causal || kw <= q + diag);
            pv = vis ? pv : 0.f;
          }
          s[qb][4 * rg + e] = pv;
          dp[qb][4 * rg + e] = pv * (dp[qb][4 * rg + e] - dd[e]);
        }
      }
    // P^T and dS^T as A operands: rows = keys, k-elements = queries in register order
    u32x4_t pa[2][2], da[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          pa[qb][h2][w] = pack_bf16(s[qb][8 * h2 + 2 * w], s[qb][8 * h2 + 2 * w + 1]);
          da[qb][h2][w] = pack_bf16(dp[qb][8 * h2 + 2 * w], dp[qb][8 * h2 + 2 * w + 1]);
        }

    // (3) dS^T into LDS (double buffered): row = key, 4 consecutive queries per write
    {
      unsigned char* dsw = dsbuf + (it & 1) * T::DSBYTES + kwl * T::DS_ROWB + 8 * hi;
      const int sw = swz_ds(kwl);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int a = 0; a < 4; ++a)
          *reinterpret_cast<u32x2_t*>(dsw + 16 * ((4 * qb + a) ^ sw)) =
              u32x2_t{da[qb][a >> 1][2 * (a & 1)], da[qb][a >> 1][2 * (a & 1) + 1]};
    }

    // (4) dV += P^T dO and dK += dS^T Q; k-step ts = 2 qb + h2 holds queries
    //     16 ts + 8 (e/4) + 4 hi + e%4, which the transposing reads of dO and Q reproduce
#pragma unroll
    for (int d0 = 0; d0 < T::DB; d0 += 2) {
      u32x2_t o[2][4][2], q[2][4][2];
#pragma unroll
      for (int dd = 0; dd < 2; ++dd)
#pragma unroll
        for (int ts = 0; ts < 4; ++ts)
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const int row = 16 * ts + 8 * r + vrow;
            const uint32_t off = ring_addr + slot * T::SLOT + 16 * ts * T::ROWB +
                                 tr_off(T::ROWB, r, d0 + dd, T::swz(row));
            lds_read_tr16x2<0, T::QBYTES>(q[dd][ts][r], o[dd][ts][r], off);
          }
#pragma unroll
      for (int dd = 0; dd < 2; ++dd) {
        lds_wait_tr(o[dd][0][0], o[dd][0][1], o[dd][1][0], o[dd][1][1]);
        lds_wait_tr(o[dd][2][0], o[dd][2][1], o[dd][3][0], o[dd][3][1]);
        lds_wait_tr(q[dd][0][0], q[dd][0][1], q[dd][1][0], q[dd][1][1]);
        lds_wait_tr(q[dd][2][0], q[dd][2][1], q[dd][3][0], q[dd][3][1]);
      }
#pragma unroll
      for (int dd = 0; dd < 2; ++dd)
#pragma unroll
        for (int ts = 0; ts < 4; ++ts) {
          const int d = d0 + dd;
          dv[d] = mfma32(pa[ts >> 1][ts & 1],
                         u32x4_t{o[dd][ts][0][0], o[dd][ts][0][1], o[dd][ts][1][0], o[dd][ts][1][1]}, dv[d]);
          dk[d] = mfma32(da[ts >> 1][ts & 1],
                         u32x4_t{q[dd][ts][0][0], q[dd][ts][0][1], q[dd][ts][1][0], q[dd][ts][1][1]}, dk[d]);
        }
    }

    wait_ring();         // tile it + 1 has landed (only tile it + 2 may be in flight)
    FA_WAIT_LGKMCNT0();  // this wave's dS^T rows are written, its ring reads done
    FA_BARRIER();

    // (5) dQ[:, 32 dsl ..) += dS K over the tile's 128 keys, for this wave's row blocks;
    //     every transposing read of dS is issued before the first wait
    {
      u32x2_t lo[QBW][BC / 16], up[QBW][BC / 16];
      const uint32_t base = ds_addr + (it & 1) * T::DSBYTES;
#pragma unroll
      for (int qq = 0; qq < QBW; ++qq)
#pragma unroll
        for (int ks = 0; ks < BC / 16; ++ks) {
          const uint32_t bk = base + 16 * ks * T::DS_ROWB;
          lds_read_tr16<0>(lo[qq][ks], bk + tr_off(T::DS_ROWB, 0, qb0 + qq, swz_ds(16 * ks + vrow)));
          lds_read_tr16<0>(up[qq][ks], bk + tr_off(T::DS_ROWB, 1, qb0 + qq, swz_ds(16 * ks + 8 + vrow)));
        }
#pragma unroll
      for (int qq = 0; qq < QBW; ++qq)
#pragma unroll
        for (int ks = 0; ks < BC / 16; ks += 2)
          lds_wait_tr(lo[qq][ks], up[qq][ks], lo[qq][ks + 1], up[qq][ks + 1]);
#pragma unroll
      for (int qq = 0; qq < QBW; ++qq) {
        const int qb = qb0 + qq;
        f32x16_t dq = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < BC / 16; ++ks)
          dq = mfma32(u32x4_t{lo[qq][ks][0], lo[qq][ks][1], up[qq][ks][0], up[qq][ks][1]}, ktf[ks], dq);
        float* dqa = p.dq_acc + (((int64_t)b * p.Hq + hq) * p.Nq + q0 + 32 * qb) * D + 32 * dsl + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ql = 8 * (r >> 2) + 4 * hi + (r & 3);
          if (q0 + 32 * qb + ql < p.Nq) unsafeAtomicAdd(dqa + (int64_t)ql * D, dq[r]);
        }
      }
    }
  }

  // ---- dK = scale * acc, dV = acc, rounded to bf16; rows >= Nk are not stored (rows in
  //      [Lk, Nk) hold zeros).  Column d = 32 blk + l32, register r holds key
  //      8 (r/4) + 4 hi + r%4 of this wave's 32 keys.
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
  e = launch(bwd_main_kernel<D>, (int64_t)p.nkt * p.Hkv * p.B, 64 * kBwdWaves, p, stream);
  if (e != hipSuccess) return e;
  return launch(bwd_dq_kernel<D>, (rows * (D / 8) + 255) / 256, 256, p, stream);
}

size_t stats_bytes(int B, int Hq, int Nq) { return ((size_t)B * Hq * Nq * 8 + 255) & ~size_t(255); }

}  // namespace

size_t bwd_workspace_bytes(int B, int Hq, int Nq, int D) {
  const size_t rows = (size_t)B * Hq * Nq;
  return stats_bytes(B, Hq, Nq) + ((rows * D * 4 + 255) & ~size_t(255));
}

void bwd_bind_workspace(BwdParams& p, void* workspace, int D) {
  (void)D;
  p.stats = static_cast<float*>(workspace);
  p.dq_acc = reinterpret_cast<float*>(static_cast<char*>(workspace) + stats_bytes(p.B, p.Hq, p.Nq));
}

hipError_t launch_bwd(const BwdParams& p, int D, hipStream_t stream) {
  return D == 128 ? launch_all<128>(p, stream) : launch_all<64>(p, stream);
}

}  // namespace fa
