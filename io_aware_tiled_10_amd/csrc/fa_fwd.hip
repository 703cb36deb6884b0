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
//  * one workgroup = 8 waves = 256 query rows, one workgroup per compute unit (two
//    waves per SIMD); each wave owns 32 rows outright (the article's "Warp级并行"
//    principle: no reduction across waves).  A K/V block staged in LDS serves all 256
//    rows, halving the L2 -> LDS traffic per FLOP against 128-row tiles.  The rows are
//    256 rows of one head, or, for a causal GQA group, 64 rows of 4 heads (128 of 2)
//    that share the K/V head, so a tile on the diagonal stops sooner;
//  * K/V blocks of 64 keys go from L2/HBM straight into LDS (LDS DMA: coalesced 1 KiB
//    per wave instruction, no staging registers) through four-slot rings, with the
//    16-byte slots of every row XOR-swizzled so that the operand reads are free of
//    bank conflicts.  K runs one block ahead of V; each load has two blocks of compute
//    to land, and one barrier per block orders the ring.  The block loop is unrolled
//    over the four slots so that every LDS operand address is a per-lane register plus
//    an immediate offset;
//  * the scores are computed transposed, S^T = K Q^T, on 32x32x16 bf16 MFMA, so each
//    lane holds one query's scores: the row max / sum are lane-local plus a single
//    exchange between the two wave halves;
//  * software pipeline inside each wave: the MFMAs of the next block's scores are
//    issued together with the exp / rescale work of the current block, which only
//    needs the vector units;
//  * the probabilities stay in registers as the B operand of O^T += V^T P^T; the V^T
//    operand comes from transposing LDS reads (ds_read_b64_tr_b16) in the key order of
//    the score registers, so no shuffle is needed between the two products;
//  * exp is exp2 with scale*log2(e) folded into one fma per score.  The exponent
//    reference is a running maximum that is moved lazily: a block's probabilities are
//    first taken against the current reference, and only if some lane's block sum
//    exceeds 2^8 (always on the first block) are the scores recomputed and the row
//    maximum, the reference and the rescale done; the common path has no max at all;
//  * causal: blocks above the diagonal are never visited, the mask is applied only
//    on blocks that cross it, and the heaviest query tiles are launched first;
//  * workgroups are ordered so tiles that share a KV head run on the same XCD;
//  * a packed batch of variable-length sequences (self-test page, section C) runs the
//    same kernel: each workgroup takes its sequence's row range from the offsets, and
//    tiles past a short sequence exit at once;
//  * FP8 Q K^T (V2/V3 article, section FP8低精度): Q and K arrive as E4M3 codes with one
//    step per 64-row block; S^T = K Q^T runs on the 32x32x64 E4M3 MFMA with fp32
//    accumulation (half the bf16 product's time), K blocks are staged at one byte per
//    element, and the two blocks' steps fold into the exp2 coefficient of each block, so
//    the softmax, P V and the epilogue are those of the bf16 path.
#include <type_traits>

#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kFwdWaves = 8;
constexpr int kFwdBR = 32 * kFwdWaves;  // query rows per workgroup
constexpr int kFwdBC = 64;              // keys per block
constexpr int kFwdSlots = 4;            // ring depth for K and for V

// QK8: K (and Q) are E4M3 codes, one byte per element; V stays bf16.
template <int D, bool QK8 = false>
struct FwdTile {
  static constexpr int KS = D / 16;              // k-steps of S^T = K Q^T (bf16)
  static constexpr int KS8 = D / 64;             // k-steps of S^T = K Q^T (E4M3)
  static constexpr int DB = D / 32;              // 32-row blocks of O^T
  static constexpr int ROWB = D * 2;             // bytes per V row
  static constexpr int SPR = D / 8;              // 16-byte slots per V row
  static constexpr int RPB = 256 / ROWB;         // V rows per 256-byte LDS bank period
  static constexpr int RPI = 1024 / ROWB;        // V rows per wave DMA instruction
  static constexpr int KROWB = QK8 ? D : 2 * D;  // bytes per staged K row
  static constexpr int KSPR = KROWB / 16;
  static constexpr int KRPB = 256 / KROWB;
  static constexpr int KRPI = 1024 / KROWB;
  static constexpr int TBYTES = kFwdBC * ROWB;   // one V block in LDS
  static constexpr int KTBYTES = kFwdBC * KROWB; // one K block in LDS
  static constexpr int NDMA = TBYTES / (1024 * kFwdWaves);    // V DMA instructions per thread
  static constexpr int NDMA_K = KTBYTES / (1024 * kFwdWaves); // K DMA instructions per thread
  static constexpr int LDS_BYTES = kFwdSlots * (KTBYTES + TBYTES);
  static_assert(NDMA * 1024 * kFwdWaves == TBYTES, "a block must split evenly over the waves");
  static_assert(NDMA_K * 1024 * kFwdWaves == KTBYTES, "a block must split evenly over the waves");
  static __device__ __forceinline__ int swz_k(int r) { return (r / KRPB) % KSPR; }
  static __device__ __forceinline__ int swz_v(int r) { return 4 * ((r / RPB) % (SPR / 4)); }
};

// A ring slot known at compile time, so that LDS addresses of a slot are immediate
// offsets from per-lane base registers.
template <int N>
struct Slot {
  static constexpr int value = N;
};

// The exponent reference m (a running maximum of the scores seen so far) is moved
// only when some lane's probability sum over one block exceeds this bound, so every
// probability stays at most 2^8: bf16 P and the fp32 sums absorb that, while the row
// maximum and almost every accumulator rescale are skipped.  The final O = acc / l and
// LSE = m*scale + ln(l) use the same reference, so the result does not depend on it.
constexpr float kMaxBlockSum = 256.f;

template <int D, bool OUT_F32, bool QK8, bool DROP = false>
__global__ void __launch_bounds__(64 * kFwdWaves) __attribute__((amdgpu_waves_per_eu(2)))
fwd_bf16_kernel(FwdParams p) {
  using T = FwdTile<D, QK8>;
  static_assert(!QK8 || D == 128, "the E4M3 path is built for D = 128");
  static_assert(!(QK8 && DROP), "dropout is built for the bf16 path");
  constexpr int BC = kFwdBC, NW = kFwdWaves, NS = kFwdSlots;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[T::LDS_BYTES];
  unsigned char* kring = lds;
  unsigned char* vring = lds + NS * T::KTBYTES;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;

  // ---- which tile: the (batch entry, KV head) groups of each XCD share its L2, heavy
  // causal tiles (rank 0) go first; the KV head varies slowest over the groups, so every
  // XCD receives every batch entry and sequences of different length (packed batches)
  // spread evenly over the XCDs.  Packed batches keep each group's ranks together: their
  // rank-0 tiles are empty for all but the longest sequences.
  // A tile holds the same RT = 256 / th query rows of th query heads of one GQA group
  // (th = 1: 256 rows of one head).  Wave w takes head slot w / (8 / th) of the tile and
  // one 32-row group of its rows (below); all waves of a tile share its key range, so a
  // causal tile stops at the diagonal of its RT rows (with th = 4, 64 rows: a quarter of
  // the masked work of a 256-row tile on the diagonal).
  const int th = p.th, wph = NW / th;  // waves per head
  const int RT = 32 * wph;             // query rows per tile
  // Rows of the waves of a 256-row tile: the two waves that share a SIMD (waves w and
  // w + 4) take row groups from opposite ends of the tile, so on the diagonal, where the
  // waves of the lower rows need more key blocks than those of the upper rows, each SIMD
  // carries about the same number of (wave, block) steps.
  const int hs = wave / wph;
  const int ro = 32 * (wph == 8 ? (wave < 4 ? wave : 11 - wave) : wave % wph);
  const TileId tid8 = tile_order(blockIdx.x, gridDim.x, p.B * p.Hkv, p.nqt, p.G / th, p.cu_q == nullptr, p.gsz);
  const int gi = tid8.gi, rank = tid8.rank;
  const int b = tid8.pair % p.B;
  const int hkv = tid8.pair / p.B;
  const int qt = p.causal ? p.nqt - 1 - rank : rank;
  const int hq = hkv * p.G + gi * th + hs;  // this wave's query head

  // this batch entry's query rows and valid keys; a packed batch takes them from the
  // offsets (clamped to the packed tensors) and shifts every row index by its first row
  int nq = p.Nq, lk = p.Nk;
  int64_t qr0 = 0, kr0 = 0;
  if (p.cu_q) {
    const int a0 = min(max(p.cu_q[b], 0), p.total_q), a1 = min(max(p.cu_q[b + 1], a0), p.total_q);
    const int c0 = min(max(p.cu_k[b], 0), p.total_k), c1 = min(max(p.cu_k[b + 1], c0), p.total_k);
    nq = a1 - a0, qr0 = a0, lk = c1 - c0, kr0 = c0;
  } else if (p.kv_lens) {
    lk = p.kv_lens[b];
    lk = lk < 0 ? 0 : (lk > p.Nk ? p.Nk : lk);
  }
  const int diag = lk - nq;  // key j visible to query i iff j <= i + diag
  const int q_wg0 = qt * RT;
  if (q_wg0 >= nq) return;  // a tile past a short sequence of a packed batch (uniform)
  int kend = lk;
  if (p.causal) {
    const int lim = q_wg0 + RT + diag;  // one past the last key the tile's last row sees
    kend = lim < kend ? lim : kend;
  }
  if (kend < 0) kend = 0;
  const int nblk = (kend + BC - 1) / BC;

  const int qi = q_wg0 + ro + l32;  // this lane's query row

  if (nblk == 0) {  // no visible key for any row of the tile: O = 0, LSE = -inf
    if (qi < nq) {
      const int64_t orow0 = b * p.os0 + hq * p.os1 + (qr0 + qi) * p.os2;
      if constexpr (OUT_F32) {
        float* orow = static_cast<float*>(p.o) + orow0;
        for (int d = 4 * hi; d < D; d += 8) *reinterpret_cast<f32x4_t*>(orow + d) = f32x4_t{};
      } else {
        uint16_t* orow = static_cast<uint16_t*>(p.o) + orow0;
        for (int d = 4 * hi; d < D; d += 8) *reinterpret_cast<u32x2_t*>(orow + d) = u32x2_t{};
      }
      if (p.lse && hi == 0) p.lse[b * p.lse_sb + hq * p.lse_sh + qr0 + qi] = -INFINITY;
    }
    return;  // uniform over the workgroup
  }

  // ---- Q^T fragments (B operand), loaded once; rows past Nq read as zero.  bf16: the
  // lane's 8-element slot 2 s + hi of its query row for k-step s; E4M3: the lane's 32
  // bytes 64 s + 32 hi .. of its row for k-step s (the K operand uses the same bytes)
  u32x4_t qf[QK8 ? 1 : T::KS];
  i32x8_t qf8[QK8 ? T::KS8 : 1];
  float dqw = 1.f;  // E4M3: the step of this wave's 64-row query block
  {
    const int64_t qpitch = p.qs2 * (QK8 ? 1 : 2);
    // this wave's 32 rows of its head (rows past Nq read as zero)
    const unsigned char* qtile = reinterpret_cast<const unsigned char*>(p.q) +
                                 (b * p.qs0 + hq * p.qs1 + (qr0 + q_wg0 + ro) * p.qs2) * (QK8 ? 1 : 2);
    const auto rq = make_rsrc(qtile, rows_span(min(32, nq - q_wg0 - ro), qpitch, T::KROWB));
    if constexpr (QK8) {
      const uint32_t off = (uint32_t)(l32 * qpitch) + 32 * hi;
#pragma unroll
      for (int s = 0; s < T::KS8; ++s)
        qf8[s] = cat8(buf_load16(rq, off + 64 * s), buf_load16(rq, off + 64 * s + 16));
      // (a wave whose rows all lie past Nq takes the last block's step; its rows are
      // never stored)
      const int qblk = min((q_wg0 + ro) / 64, (nq + 63) / 64 - 1);
      dqw = p.q_scale[b * p.qsc_b + hq * p.qsc_h + qblk];
    } else {
      const uint32_t off = (uint32_t)(l32 * qpitch) + 16 * hi;
#pragma unroll
      for (int s = 0; s < T::KS; ++s) qf[s] = buf_load16(rq, off + 32 * s);
    }
    asm volatile("" ::: "memory");  // issue these before the ring loads below
  }

  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(p.k) +
                               (b * p.ks0 + hkv * p.ks1 + kr0 * p.ks2) * (QK8 ? 1 : 2);
  const uint16_t* vbase = p.v + b * p.vs0 + hkv * p.vs1 + kr0 * p.vs2;
  const int64_t kpitch = p.ks2 * (QK8 ? 1 : 2), vpitch = p.vs2 * 2;

  // DMA: thread (wave w, lane) fills, for instruction i, row RPI (NW i + w) + lane / SPR,
  // slot lane % SPR, with the swizzled 16-byte chunk of that row; the swizzle of that
  // row does not depend on i, and the row step of i goes into the scalar offset.
  const int drow = T::RPI * wave + lane / T::SPR, dslot = lane % T::SPR;
  const int krow_d = T::KRPI * wave + lane / T::KSPR, kslot_d = lane % T::KSPR;
  const uint32_t kdma = (uint32_t)(krow_d * kpitch) + 16 * (kslot_d ^ T::swz_k(krow_d));
  const uint32_t vdma = (uint32_t)(drow * vpitch) + 16 * (dslot ^ T::swz_v(drow));
  const int kstep = (int)(NW * T::KRPI * kpitch), vstep = (int)(NW * T::RPI * vpitch);

  auto dma_k = [&](int blk, int slot) {  // blocks past the keys fill the slot with zeros
    const int key0 = blk * BC;
    const auto rk = make_rsrc(kbase + (int64_t)key0 * kpitch, rows_span(min(BC, lk - key0), kpitch, T::KROWB));
    unsigned char* dst = kring + slot * T::KTBYTES + 1024 * wave;
#pragma unroll
    for (int i = 0; i < T::NDMA_K; ++i) lds_dma16(rk, dst + 1024 * NW * i, kdma, 0, kstep * i);
  };
  auto dma_v = [&](int blk, int slot) {
    const int key0 = blk * BC;
    const auto rv = make_rsrc(vbase + (int64_t)key0 * p.vs2, rows_span(min(BC, lk - key0), vpitch, D * 2));
    unsigned char* dst = vring + slot * T::TBYTES + 1024 * wave;
#pragma unroll
    for (int i = 0; i < T::NDMA; ++i) lds_dma16(rv, dst + 1024 * NW * i, vdma, 0, vstep * i);
  };

  // S^T operand reads: rows l32 and 32 + l32 (same swizzle); bf16: logical slot
  // 2 ks + hi; E4M3: logical slots 4 s + 2 hi and 4 s + 2 hi + 1 (32 bytes)
  const int krow = l32 * T::KROWB, ksw = T::swz_k(l32);
  auto qk = [&](int slot, f32x16_t& s0, f32x16_t& s1) {
    const unsigned char* ks = kring + slot * T::KTBYTES + krow;
    s0 = f32x16_t{};
    s1 = f32x16_t{};
    if constexpr (QK8) {
#pragma unroll
      for (int k = 0; k < T::KS8; ++k) {
        const int o0 = 16 * ((4 * k + 2 * hi) ^ ksw), o1 = 16 * ((4 * k + 2 * hi + 1) ^ ksw);
        const i32x8_t a0 = cat8(*reinterpret_cast<const u32x4_t*>(ks + o0),
                                *reinterpret_cast<const u32x4_t*>(ks + o1));
        const i32x8_t a1 = cat8(*reinterpret_cast<const u32x4_t*>(ks + 32 * T::KROWB + o0),
                                *reinterpret_cast<const u32x4_t*>(ks + 32 * T::KROWB + o1));
        s0 = mfma32_f8(a0, qf8[k], s0);
        s1 = mfma32_f8(a1, qf8[k], s1);
      }
    } else {
#pragma unroll
      for (int k = 0; k < T::KS; ++k) {
        const int o = 16 * ((2 * k + hi) ^ ksw);
        const u32x4_t a0 = *reinterpret_cast<const u32x4_t*>(ks + o);
        const u32x4_t a1 = *reinterpret_cast<const u32x4_t*>(ks + 32 * T::KROWB + o);
        s0 = mfma32(a0, qf[k], s0);
        s1 = mfma32(a1, qf[k], s1);
      }
    }
  };

  // V^T operand reads (transposing): lane 16 g + i reads row 16 ts + 8 r + 4 (g/2) + i/4,
  // columns 32 db + 16 (g%2) + 4 (i%4) .. +3; the row's swizzle depends only on i.
  const int vg = lane >> 4, vi = lane & 15;
  const int vrow = 4 * (vg >> 1) + (vi >> 2);
  const int vsw = T::swz_v(vrow) >> 2;
  const uint32_t vlane = vrow * T::ROWB + 16 * (2 * (vg & 1) + ((vi & 3) >> 1)) + 8 * (vi & 1);
  uint32_t vaddr[T::DB];  // per 32-column block of V, slot 0
#pragma unroll
  for (int d = 0; d < T::DB; ++d) vaddr[d] = lds_addr(vring) + vlane + 64 * (d ^ vsw);

  f32x16_t acc[T::DB];
#pragma unroll
  for (int d = 0; d < T::DB; ++d) acc[d] = f32x16_t{};
  float m = -INFINITY, l = 0.f;  // m: exponent reference (unscaled q.k units)
  const float c = p.scale_log2;
  // E4M3: the MFMA gives q_hat.k_hat; a block's scores are that times dqw * (its key
  // block's step).  The steps are read one block ahead with scalar loads.
  const auto* kscl = (const __attribute__((address_space(4))) float*)(
      QK8 ? p.k_scale + b * p.ksc_b + hkv * p.ksc_h : p.k_scale);
  float dk_next = QK8 ? kscl[0] : 1.f;

  // One block: (s0, s1) hold the scores of block j (keys 64 j + [0, 32), + [32, 64));
  // the scores of block j + 1 are produced into (n0, n1).
  // `slot` is j % NS.
  // `act`: false when every key of block j lies past the diagonal of all of this wave's
  // rows (only in the steps after the unrolled loop, where the tile's last blocks cross
  // the diagonal): the wave then skips the block's work, whose probabilities would all
  // be exactly zero, and only issues its share of the ring loads and meets the barrier.
  auto step = [&](int j, auto slot, f32x16_t& s0, f32x16_t& s1, f32x16_t& n0, f32x16_t& n1,
                  auto first, bool act) {
    constexpr int sl = decltype(slot)::value;
    constexpr bool kFirst = decltype(first)::value;
    constexpr uint32_t vo = sl * T::TBYTES;
    // K_{j+3} and V_{j+2} into the slots of K_{j-1} and V_{j-2}, which are free
    dma_k(j + 3, (sl + 3) % NS);
    dma_v(j + 2, (sl + 2) % NS);
    if (act) {
    float sq = 1.f;  // score units per MFMA unit of this block
    if constexpr (QK8) {
      sq = dqw * dk_next;
      dk_next = kscl[min(j + 1, nblk - 1)];
    }
    const float cb = c * sq;

    const int key0 = j * BC;
    const bool edge = (key0 + BC > lk) || (p.causal && key0 + BC - 1 > q_wg0 + diag);
    auto mask = [&](f32x16_t& a0, f32x16_t& a1) {
      if (edge) {
        const int last = p.causal ? min(lk - 1, qi + diag) : lk - 1;  // last visible key
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (key > last) a0[r] = -INFINITY;
          if (key + 32 > last) a1[r] = -INFINITY;
        }
      }
    };
    mask(s0, s1);

    // next block's scores on the matrix cores while this block's exps run on the VALU
    // (past the last block the slot holds zeros and the result is not used)
    qk((sl + 1) % NS, n0, n1);

    // probabilities against the current reference, packed to bf16 as the B operand of
    // the second product; returns this lane's sum of them
    u32x4_t pf[4];
    // dropout: the mask bytes of this lane's 16 keys of each half (register r <-> byte
    // r); the sum l keeps every probability, P V only the kept ones (the 1 / keep factor
    // is applied with 1 / l at the end)
    u32x4_t zw0{}, zw1{};
    if constexpr (DROP) {
      zw0 = dropout_words(key0 / 32, hi, qi, hq, b, p.seed_lo, p.seed_hi);
      zw1 = dropout_words(key0 / 32 + 1, hi, qi, hq, b, p.seed_lo, p.seed_hi);
    }
    auto probs = [&](const f32x16_t& a0, const f32x16_t& a1) {
      const float mc = (m == -INFINITY ? 0.f : m) * c;
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(fmaf(a0[r], cb, -mc)), p1 = fast_exp2(fmaf(a0[r + 1], cb, -mc));
        const float p2 = fast_exp2(fmaf(a1[r], cb, -mc)), p3 = fast_exp2(fmaf(a1[r + 1], cb, -mc));
        rs += (p0 + p1) + (p2 + p3);
        if constexpr (DROP) {
          const uint32_t t = p.drop_t;
          pf[r >> 3][(r & 7) >> 1] =
              pack_bf16(dropout_keep(zw0[r >> 2], r & 3, t) ? p0 : 0.f,
                        dropout_keep(zw0[(r + 1) >> 2], (r + 1) & 3, t) ? p1 : 0.f);
          pf[2 + (r >> 3)][(r & 7) >> 1] =
              pack_bf16(dropout_keep(zw1[r >> 2], r & 3, t) ? p2 : 0.f,
                        dropout_keep(zw1[(r + 1) >> 2], (r + 1) & 3, t) ? p3 : 0.f);
        } else {
          pf[r >> 3][(r & 7) >> 1] = pack_bf16(p0, p1);
          pf[2 + (r >> 3)][(r & 7) >> 1] = pack_bf16(p2, p3);
        }
      }
      return rs;
    };
    float rs = probs(s0, s1);
    // The reference is kept while every lane's block sum stays within the bound (so
    // no probability exceeds it).  Otherwise -- and always on the first block, where
    // there is no reference yet -- the scores are recomputed from the K block still in
    // its slot, the reference moves to the row maximum, and the running sum and the
    // accumulator are rescaled.  The test also catches inf and NaN sums.
    if (kFirst || __builtin_amdgcn_ballot_w64(!(rs <= kMaxBlockSum))) {
      asm volatile("" ::: "memory");  // keep this path's LDS reads off the common path
      qk(sl, s0, s1);
      mask(s0, s1);
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(fmaxf(mx, s0[r]), s1[r]);
      mx = halves_max(mx) * sq;
      const float m_new = fmaxf(m, mx);
      const float alpha = m == -INFINITY ? 0.f : fast_exp2((m - m_new) * c);
      l *= alpha;
#pragma unroll
      for (int d = 0; d < T::DB; ++d) acc[d] *= alpha;
      m = m_new;
      rs = probs(s0, s1);
    }
    l += rs;

    // O^T += V^T P^T; k-step ts holds keys 16 ts + 8 (e/4) + 4 hi + e%4 (e = 0..7)
    // the V^T reads of each 32-column block are issued before the products of the
    // previous block, so their latency hides under those products (LDS returns in
    // order: after issuing block d + 1, a count of 8 means block d has arrived)
    u32x2_t v[2][4][2];
    auto vread = [&](int d, u32x2_t (&w)[4][2]) {
      const uint32_t a = vaddr[d];
      lds_read_tr16x2<vo, vo + 8 * T::ROWB>(w[0][0], w[0][1], a);
      lds_read_tr16x2<vo + 16 * T::ROWB, vo + 24 * T::ROWB>(w[1][0], w[1][1], a);
      lds_read_tr16x2<vo + 32 * T::ROWB, vo + 40 * T::ROWB>(w[2][0], w[2][1], a);
      lds_read_tr16x2<vo + 48 * T::ROWB, vo + 56 * T::ROWB>(w[3][0], w[3][1], a);
    };
    vread(0, v[0]);
#pragma unroll
    for (int d = 0; d < T::DB; ++d) {
      u32x2_t (&w)[4][2] = v[d & 1];
      if (d + 1 < T::DB) {
        vread(d + 1, v[(d + 1) & 1]);
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
    }  // act

    // the loads of blocks j + 2 (K) and j + 1 (V), issued one block ago, have landed
    // (only this block's may still be in flight); the barrier then publishes them and
    // frees the slots this block read
    wait_vmcnt<T::NDMA + T::NDMA_K>();
    FA_WAIT_LGKMCNT0();
    FA_BARRIER();
  };
  static_assert(T::NDMA == 2 || T::NDMA == 1, "wait counts above assume D = 128 or 64");

  dma_k(0, 0);
  dma_k(1, 1);
  dma_k(2, 2);
  dma_v(0, 0);
  dma_v(1, 1);
  FA_WAIT_VMCNT(0);
  __syncthreads();
  f32x16_t sa0, sa1, sb0, sb1;
  qk(0, sa0, sa1);
  FA_WAIT_LGKMCNT0();  // K slot 0 is refilled at the top of the first block:
  __syncthreads();     // every wave's reads of it must be done

  // The first block (which sets the reference) is peeled off, so the loop body carries
  // no test of j and its exps can be scheduled between the next block's MFMAs.  NS
  // blocks per trip, so every slot index is a constant; the score registers alternate.
  static_assert(NS == 4, "the unrolled loop below walks four slots");
  using Later = std::false_type;
  step(0, Slot<0>{}, sa0, sa1, sb0, sb1, std::true_type{}, true);
  int j = 1;
  for (; j + 3 < nblk; j += 4) {
    step(j, Slot<1>{}, sb0, sb1, sa0, sa1, Later{}, true);
    step(j + 1, Slot<2>{}, sa0, sa1, sb0, sb1, Later{}, true);
    step(j + 2, Slot<3>{}, sb0, sb1, sa0, sa1, Later{}, true);
    step(j + 3, Slot<0>{}, sa0, sa1, sb0, sb1, Later{}, true);
  }
  // the last block any row of this wave sees (causal; a wave whose rows see no key
  // keeps to the first block)
  const int wlast = p.causal ? max(q_wg0 + ro + 31 + diag, 0) / BC : nblk - 1;
  if (j < nblk) step(j, Slot<1>{}, sb0, sb1, sa0, sa1, Later{}, j <= wlast);
  if (j + 1 < nblk) step(j + 1, Slot<2>{}, sa0, sa1, sb0, sb1, Later{}, j + 1 <= wlast);
  if (j + 2 < nblk) step(j + 2, Slot<3>{}, sb0, sb1, sa0, sa1, Later{}, j + 2 <= wlast);
  FA_WAIT_VMCNT(0);  // the trailing loads (past the keys: zeros) write the ring too

  // ---- epilogue: O = acc / l once (times 1 / keep with dropout); LSE = m * scale + ln(l).
  // l == 0 only when no key was visible (O = 0, LSE = -inf); a NaN l (a NaN score) stays
  // NaN in O and LSE
  const float lt = halves_sum(l);
  const float inv = lt == 0.f ? 0.f : (DROP ? p.drop_scale : 1.f) / lt;
  if (qi < nq) {
    const int64_t orow0 = b * p.os0 + hq * p.os1 + (qr0 + qi) * p.os2;
    if constexpr (OUT_F32) {
      float* orow = static_cast<float*>(p.o) + orow0;
#pragma unroll
      for (int d = 0; d < T::DB; ++d)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg)
          *reinterpret_cast<f32x4_t*>(orow + 32 * d + 8 * rg + 4 * hi) =
              f32x4_t{acc[d][4 * rg] * inv, acc[d][4 * rg + 1] * inv, acc[d][4 * rg + 2] * inv,
                      acc[d][4 * rg + 3] * inv};
    } else {
      uint16_t* orow = static_cast<uint16_t*>(p.o) + orow0;
#pragma unroll
      for (int d = 0; d < T::DB; ++d)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg)
          *reinterpret_cast<u32x2_t*>(orow + 32 * d + 8 * rg + 4 * hi) =
              u32x2_t{pack_bf16(acc[d][4 * rg] * inv, acc[d][4 * rg + 1] * inv),
                      pack_bf16(acc[d][4 * rg + 2] * inv, acc[d][4 * rg + 3] * inv)};
    }
    if (p.lse && hi == 0)
      p.lse[b * p.lse_sb + hq * p.lse_sh + qr0 + qi] = lt == 0.f ? -INFINITY : m * p.scale + __logf(lt);
  }
}

// fp32 inputs, D = 64: one lane per query row, K/V blocks of 32 keys broadcast from
// LDS, fp32 FMA on the vector units (the small fp32 workload is latency-bound; the
// matrix cores are reserved for the bf16 path).  The NW waves of a workgroup share its
// 64 query rows and split the key blocks among them (wave w takes blocks w, w + NW, ...,
// each through its own LDS buffers), each keeping its own running (m, l, acc); at the
// end the NW partial states of each row are merged through LDS by the LSE rule (the
// same rule the split-KV decode merge applies), each wave finishing D / NW columns.
constexpr int kF32BR = 64, kF32BC = 32, kF32Waves = 8;

template <int D, int NW>
__global__ void __launch_bounds__(64 * NW) fwd_f32_kernel(FwdParams p) {
  static_assert(D % NW == 0, "the merge splits the columns evenly over the waves");
  // K and V blocks of each wave; after the key loop the same memory holds the waves'
  // accumulators, [wave][column][row]
  __shared__ __attribute__((aligned(16))) float kvbuf[NW][2][kF32BC][D];
  __shared__ float mlbuf[2][NW][kF32BR];
  static_assert(sizeof(kvbuf) >= sizeof(float) * NW * D * kF32BR, "merge area");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

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
  const int nblk = (kend + kF32BC - 1) / kF32BC;
  const int qi = q_wg0 + lane;
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
  float (*ks)[D] = kvbuf[wave][0];
  float (*vs)[D] = kvbuf[wave][1];

  // every wave runs the same number of trips (the barriers are shared); a trip past the
  // wave's last block loads and computes nothing
  const int trips = (nblk + NW - 1) / NW;
  for (int it = 0; it < trips; ++it) {
    const int blk = it * NW + wave;
    const int key0 = blk * kF32BC;
    const bool live = blk < nblk;
    __syncthreads();  // the previous trip's reads of this wave's buffers are done
    if (live) {
      for (int e = lane; e < kF32BC * D / 4; e += 64) {
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
    }
    __syncthreads();
    if (!live) continue;
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

  // ---- merge: wave w's state of row `lane` -> LDS; wave w then finishes columns
  //      [w D / NW, (w + 1) D / NW) of every row: M = max_w m_w, a_w = 2^((m_w - M) c)
  //      (0 for a wave that saw no key), L = sum_w a_w l_w, O = sum_w a_w acc_w / L,
  //      LSE = M scale + ln L (O = 0, LSE = -inf when L = 0)
  __syncthreads();
  float* accbuf = &kvbuf[0][0][0][0];
#pragma unroll
  for (int d = 0; d < D; ++d) accbuf[(wave * D + d) * kF32BR + lane] = acc[d];
  mlbuf[0][wave][lane] = m;
  mlbuf[1][wave][lane] = l;
  __syncthreads();
  float mw[NW], M = -INFINITY;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    mw[w] = mlbuf[0][w][lane];
    M = fmaxf(M, mw[w]);
  }
  float aw[NW], L = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    aw[w] = mw[w] == -INFINITY ? 0.f : fast_exp2((mw[w] - M) * c);
    L += aw[w] * mlbuf[1][w][lane];
  }
  if (qi < p.Nq) {
    const float inv = L == 0.f ? 0.f : 1.f / L;
    constexpr int DC = D / NW;
    const int d0 = wave * DC;
    float* orow = static_cast<float*>(p.o) + b * p.os0 + hq * p.os1 + (int64_t)qi * p.os2;
#pragma unroll
    for (int d = 0; d < DC; d += 4) {
      f32x4_t o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) x = fmaf(aw[w], accbuf[(w * D + d0 + d + e) * kF32BR + lane], x);
        o[e] = x * inv;
      }
      *reinterpret_cast<f32x4_t*>(orow + d0 + d) = o;
    }
    if (p.lse && wave == 0)
      p.lse[b * p.lse_sb + hq * p.lse_sh + qi] = L == 0.f ? -INFINITY : M * p.scale + __logf(L);
  }
}

// fp32 forward for small grids (fewer 64-row tiles than two per compute unit, as in the
// B1 H2 N256 workload, where the kernel above would leave all but a few compute units idle):
// a workgroup of 256 threads takes a tile of TR = 16 query rows, and thread (row r, subset s)
// keeps the running (m, l, acc) of row r over the keys j = s (mod NS), NS = 16, so each row's
// work is spread over 16 threads and the grid has four times as many workgroups.  K and V
// come through LDS in chunks of KC = 128 keys, each row padded by 16 bytes so that the keys a
// wave reads at once lie in different banks.  At the end the NS partial states of each row
// are merged through LDS by the LSE rule, thread (r, s) finishing columns D / NS * s .. of
// row r.
constexpr int kF32SmallThreads = 256, kF32SmallBR = 16, kF32KC = 128;

template <int D>
__global__ void __launch_bounds__(kF32SmallThreads) fwd_f32_small_kernel(FwdParams p) {
  constexpr int TR = kF32SmallBR, NS = kF32SmallThreads / TR, KC = kF32KC, RP = D + 4, KI = KC / NS, CW = D / NS;
  constexpr int NLD = KC * D / 4 / kF32SmallThreads;  // 16-byte loads per thread per tensor and chunk
  static_assert(CW % 4 == 0 && KC % NS == 0 && NLD * 4 * kF32SmallThreads == KC * D, "tile shape");
  // K and V chunks; after the key loop the same memory holds the threads' accumulators,
  // subset s at [s * SD], column d, row r at [s * SD + d * TR + r]
  constexpr int SD = D * TR + 4;
  __shared__ __attribute__((aligned(16))) float kv[2][KC][RP];
  __shared__ float mlbuf[2][NS][TR];
  static_assert(sizeof(kv) >= sizeof(float) * NS * SD, "merge area");
  const int tid = threadIdx.x;
  const int r = tid % TR, s = tid / TR;

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
  const int q_wg0 = qt * TR;
  int kend = lk;
  if (p.causal) {
    const int lim = q_wg0 + TR + diag;
    kend = lim < kend ? lim : kend;
  }
  if (kend < 0) kend = 0;
  const int qi = q_wg0 + r;
  const int last = p.causal ? min(lk - 1, qi + diag) : lk - 1;

  const float* qsrc = static_cast<const float*>(static_cast<const void*>(p.q));
  const float* ksrc = static_cast<const float*>(static_cast<const void*>(p.k)) + b * p.ks0 + hkv * p.ks1;
  const float* vsrc = static_cast<const float*>(static_cast<const void*>(p.v)) + b * p.vs0 + hkv * p.vs1;

  float q[D], acc[D];
  const float c = p.scale_log2;
  const float* qrow = qsrc + b * p.qs0 + hq * p.qs1 + (int64_t)qi * p.qs2;
#pragma unroll
  for (int d = 0; d < D; d += 4) {
    const f32x4_t v4 = qi < p.Nq ? *reinterpret_cast<const f32x4_t*>(qrow + d) : f32x4_t{};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      q[d + e] = v4[e];
      acc[d + e] = 0.f;
    }
  }
  float m = -INFINITY, l = 0.f;

  for (int c0 = 0; c0 < kend; c0 += KC) {
    // the chunk's loads are all issued before any is stored, so their latencies overlap
    f32x4_t k4[NLD], v4[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int e = tid + kF32SmallThreads * i;
      const int key = c0 + e / (D / 4), col = 4 * (e % (D / 4));
      k4[i] = v4[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (key < lk) {
        k4[i] = *reinterpret_cast<const f32x4_t*>(ksrc + (int64_t)key * p.ks2 + col);
        v4[i] = *reinterpret_cast<const f32x4_t*>(vsrc + (int64_t)key * p.vs2 + col);
      }
    }
    __syncthreads();  // the previous chunk's reads are done
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int e = tid + kF32SmallThreads * i;
      const int row = e / (D / 4), col = 4 * (e % (D / 4));
      *reinterpret_cast<f32x4_t*>(&kv[0][row][col]) = k4[i];
      *reinterpret_cast<f32x4_t*>(&kv[1][row][col]) = v4[i];
    }
    __syncthreads();
    // this thread's keys of the chunk: rows s, s + NS, ..., each against query row qi
    float sc[KI];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int row = s + NS * i;
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < D; d += 4) {
        const f32x4_t k4 = *reinterpret_cast<const f32x4_t*>(&kv[0][row][d]);
#pragma unroll
        for (int e = 0; e < 4; ++e) dot = fmaf(q[d + e], k4[e], dot);
      }
      sc[i] = c0 + row > last ? -INFINITY : dot;
      mx = fmaxf(mx, sc[i]);
    }
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2((m - m_use) * c);
    const float mc = m_use * c;
    l *= alpha;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] *= alpha;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int row = s + NS * i;
      const float pj = fast_exp2(fmaf(sc[i], c, -mc));
      l += pj;
#pragma unroll
      for (int d = 0; d < D; d += 4) {
        const f32x4_t v4 = *reinterpret_cast<const f32x4_t*>(&kv[1][row][d]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[d + e] = fmaf(pj, v4[e], acc[d + e]);
      }
    }
    m = m_new;
  }

  // ---- merge: thread (r, s)'s state -> LDS; thread (r, s) then finishes columns CW s ..
  //      CW s + CW - 1 of row r: M = max_s' m_s', a_s' = 2^((m_s' - M) c) (0 for a subset
  //      that saw no key), L = sum_s' a_s' l_s', O = sum_s' a_s' acc_s' / L, LSE = M scale
  //      + ln L (O = 0, LSE = -inf when L = 0)
  __syncthreads();
  float* accbuf = &kv[0][0][0];
#pragma unroll
  for (int d = 0; d < D; ++d) accbuf[s * SD + d * TR + r] = acc[d];
  mlbuf[0][s][r] = m;
  mlbuf[1][s][r] = l;
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < NS; ++w) M = fmaxf(M, mlbuf[0][w][r]);
  float aw[NS], L = 0.f;
#pragma unroll
  for (int w = 0; w < NS; ++w) {
    const float mw = mlbuf[0][w][r];
    aw[w] = mw == -INFINITY ? 0.f : fast_exp2((mw - M) * c);
    L += aw[w] * mlbuf[1][w][r];
  }
  if (qi < p.Nq) {
    const float inv = L == 0.f ? 0.f : 1.f / L;
    float* orow = static_cast<float*>(p.o) + b * p.os0 + hq * p.os1 + (int64_t)qi * p.os2;
#pragma unroll
    for (int d = CW * s; d < CW * s + CW; d += 4) {
      f32x4_t o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = 0.f;
#pragma unroll
        for (int w = 0; w < NS; ++w) x = fmaf(aw[w], accbuf[w * SD + (d + e) * TR + r], x);
        o[e] = x * inv;
      }
      *reinterpret_cast<f32x4_t*>(orow + d) = o;
    }
    if (p.lse && s == 0)
      p.lse[b * p.lse_sb + hq * p.lse_sh + qi] = L == 0.f ? -INFINITY : M * p.scale + __logf(L);
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

// Tile shape of the bf16 kernels: a causal tile on the diagonal computes its whole last
// key blocks for rows that see only part of them, so with GQA (query heads sharing a KV
// head) a tile takes 64 rows of 4 heads (or 128 rows of 2) instead of 256 rows of one
// head: the same K/V blocks per tile, a quarter of the masked work.  Sets p.th and
// p.nqt; returns the workgroup count.
int64_t bf16_grid(FwdParams& p) {
  p.th = 1;
  if (p.causal) {
    if (p.G % 4 == 0) p.th = 4;
    else if (p.G % 2 == 0) p.th = 2;
  }
  const int rt = kFwdBR / p.th;
  p.nqt = (p.Nq + rt - 1) / rt;
  // (batch entry, KV head) groups an XCD works through at a time: one when every tile
  // does the same work (non-causal), else enough for two tiles per compute unit of the
  // XCD (32), so the longest-first order inside a batch of groups still balances
  const int per_pair = p.nqt * (p.G / p.th);
  p.gsz = p.causal ? (2 * 32 + per_pair - 1) / per_pair : 1;
  return (int64_t)p.nqt * (p.Hq / p.th) * p.B;
}

hipError_t launch_fwd(const FwdParams& p0, int in_dtype, int out_dtype, int D, hipStream_t stream) {
  FwdParams p = p0;
  if (in_dtype == FA_F32) {
    // 64-row tiles of eight waves when they give every compute unit two workgroups,
    // else 16-row tiles whose rows are each spread over 16 threads
    const int64_t tiles64 = (int64_t)((p.Nq + kF32BR - 1) / kF32BR) * p.Hq * p.B;
    const bool small = tiles64 < 2 * 256;
    const int tr = small ? kF32SmallBR : kF32BR;
    p.nqt = (p.Nq + tr - 1) / tr;
    const int64_t grid = (int64_t)p.nqt * p.Hq * p.B;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    return small ? launch(fwd_f32_small_kernel<64>, (int)grid, kF32SmallThreads, p, stream)
                 : launch(fwd_f32_kernel<64, kF32Waves>, (int)grid, 64 * kF32Waves, p, stream);
  }
  const int64_t grid = bf16_grid(p);
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const bool of32 = out_dtype == FA_F32;
  if (D == 128)
    return of32 ? launch(fwd_bf16_kernel<128, true, false>, (int)grid, 64 * kFwdWaves, p, stream)
                : launch(fwd_bf16_kernel<128, false, false>, (int)grid, 64 * kFwdWaves, p, stream);
  return of32 ? launch(fwd_bf16_kernel<64, true, false>, (int)grid, 64 * kFwdWaves, p, stream)
              : launch(fwd_bf16_kernel<64, false, false>, (int)grid, 64 * kFwdWaves, p, stream);
}

hipError_t launch_fwd_dropout(const FwdParams& p0, int out_dtype, int D, hipStream_t stream) {
  FwdParams p = p0;
  const int64_t grid = bf16_grid(p);
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const bool of32 = out_dtype == FA_F32;
  if (D == 128)
    return of32 ? launch(fwd_bf16_kernel<128, true, false, true>, (int)grid, 64 * kFwdWaves, p, stream)
                : launch(fwd_bf16_kernel<128, false, false, true>, (int)grid, 64 * kFwdWaves, p, stream);
  return of32 ? launch(fwd_bf16_kernel<64, true, false, true>, (int)grid, 64 * kFwdWaves, p, stream)
              : launch(fwd_bf16_kernel<64, false, false, true>, (int)grid, 64 * kFwdWaves, p, stream);
}

hipError_t launch_fwd_fp8(const FwdParams& p0, int out_dtype, hipStream_t stream) {
  FwdParams p = p0;
  const int64_t grid = bf16_grid(p);
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  return out_dtype == FA_F32
             ? launch(fwd_bf16_kernel<128, true, true>, (int)grid, 64 * kFwdWaves, p, stream)
             : launch(fwd_bf16_kernel<128, false, true>, (int)grid, 64 * kFwdWaves, p, stream);
}

}  // namespace fa
