// fa_decode.hip -- split-KV decode over a variable-length KV cache, for gfx950.
//
// Method (interview answer "flash attention呢", 高频追问 2; self-test page section F):
// during decode each sequence contributes one new query per head and the whole KV
// cache must be read, so the work is bound by HBM bandwidth.  The cache of each
// sequence is cut into chunks of `split_len` keys; every chunk is attended on its
// own (online softmax inside the chunk) giving a normalised partial output O_c and
// its log-sum-exp LSE_c; a second pass merges the chunks with the same rescaling the
// online softmax uses between blocks (study card airsota.com/?p=1562, section 三):
//   M = max_c LSE_c,  w_c = exp(LSE_c - M),  O = sum w_c O_c / sum w_c,
//   LSE = M + ln sum w_c.
//
// gfx950 mapping:
//  * one workgroup per (chunk, KV head, sequence), so every cached K/V byte is read
//    from HBM exactly once and shared by the query heads of its GQA group, which
//    occupy the 32 columns of the MFMA tile (padding columns are zero queries);
//  * each of the 4 waves walks its own 32-key blocks of the chunk (no workgroup
//    barrier in the streaming loop); keys feed S^T = K q^T straight from global
//    memory, V goes through a per-wave transposed LDS tile for O^T += V^T P^T;
//  * the four waves' (m, l, acc) are merged through LDS at the end of the chunk;
//  * chunks past a sequence's length exit at once; keys past it are never loaded.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kDecWaves = 4;
constexpr int kDecBlock = 32;  // keys per wave step

__device__ __forceinline__ int vt_pos16(int k) {
  return (k & ~15) | (((k >> 2) & 1) << 3) | (((k >> 3) & 1) << 2) | (k & 3);
}

__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D>
struct DecTile {
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int CPR = D / 8;           // 16-byte chunks per cached row
  static constexpr int NG = CPR / 8;          // column passes: 8 columns x 8 key quads each
  static constexpr int VT_LD = kDecBlock + 8;
  static constexpr int VT_ELEMS = D * VT_LD;   // per wave (bf16)
  static constexpr int MRG_FLOATS = 64 + D * 32;  // per merged wave: m, l, acc
  static constexpr int VT_BYTES = kDecWaves * VT_ELEMS * 2;
  static constexpr int MRG_BYTES = (kDecWaves - 1) * MRG_FLOATS * 4;
  static constexpr int LDS_BYTES = VT_BYTES > MRG_BYTES ? VT_BYTES : MRG_BYTES;
};

template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
decode_split_kernel(DecParams p) {
  using T = DecTile<D>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[T::LDS_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar descriptors
  const int l32 = lane & 31, hi = lane >> 5;
  const int c = blockIdx.x, s = blockIdx.z;
  const int hkv = blockIdx.y / p.nhb, hb = blockIdx.y % p.nhb;

  int L = p.seq_lens[s];
  L = L < 0 ? 0 : (L > p.max_len ? p.max_len : L);
  const int start = c * p.split_len;
  if (start >= L) return;  // uniform over the workgroup
  const int end = min(start + p.split_len, L);
  const int nb = (end - start + kDecBlock - 1) / kDecBlock;

  const int gh = hb * 32 + l32;  // head within the GQA group held by this lane's column
  const bool hvalid = gh < p.G;
  const int hq = hkv * p.G + gh;
  const u32x4_t zero4 = {0u, 0u, 0u, 0u};

  u32x4_t qf[T::KS];
  {
    const uint16_t* qrow = p.q + s * p.qs0 + (int64_t)hq * p.qs1;
#pragma unroll
    for (int k = 0; k < T::KS; ++k)
      qf[k] = hvalid ? *reinterpret_cast<const u32x4_t*>(qrow + 16 * k + 8 * hi) : zero4;
  }
  const uint16_t* kb = p.k + s * p.ks0 + hkv * p.ks1;
  const uint16_t* vb = p.v + s * p.vs0 + hkv * p.vs1;
  const int64_t kpitch = p.ks2 * 2, vpitch = p.vs2 * 2;
  uint16_t* vt = reinterpret_cast<uint16_t*>(lds) + wave * T::VT_ELEMS;
  // V staging: lanes 8j..8j+7 hold the 8 four-key groups of one 16-byte column, so the
  // transposed writes of 8 lanes fill one 32-key V^T row.
  const int vq = lane % 8, vcol0 = lane / 8;
  const float cl = p.scale_log2;
  const uint32_t koff = (uint32_t)(l32 * kpitch) + 16 * hi;
  const uint32_t voff = (uint32_t)(4 * vq * vpitch) + 16 * vcol0;

  f32x16_t acc[T::DB];
#pragma unroll
  for (int d = 0; d < T::DB; ++d) acc[d] = f32x16_t{};
  float m = -INFINITY, l = 0.f;

  // keys of this wave's block n: [start + 32 (wave + 4 n), ...); out-of-chunk rows read 0
  u32x4_t ka[2][T::KS], vr[2][T::NG][4];
  auto load = [&](int buf, int blk) {
    const int key0 = start + blk * kDecBlock;
    const int rows = min(kDecBlock, end - key0);
    const auto rk = make_rsrc(kb + (int64_t)key0 * p.ks2, rows_span(rows, kpitch, D * 2));
    const auto rv = make_rsrc(vb + (int64_t)key0 * p.vs2, rows_span(rows, vpitch, D * 2));
#pragma unroll
    for (int k = 0; k < T::KS; ++k) ka[buf][k] = buf_load16(rk, koff + 32 * k);
#pragma unroll
    for (int g = 0; g < T::NG; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vr[buf][g][i] = buf_load16(rv, voff + (uint32_t)(i * vpitch) + 16 * (T::CPR / T::NG) * g);
  };

  auto step = [&](int buf, int blk) {
    const int key0 = start + blk * kDecBlock;
    f32x16_t sc{};
#pragma unroll
    for (int k = 0; k < T::KS; ++k) sc = mfma32(ka[buf][k], qf[k], sc);
    if (key0 + kDecBlock > end) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (key0 + 8 * (r >> 2) + 4 * hi + (r & 3) >= end) sc[r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[r]);
    mx = halves_max(mx);
    const float m_new = fmaxf(m, mx);  // finite: the wave's first block holds a valid key
    const float alpha = fast_exp2((m - m_new) * cl);  // 0 on the first block, 1 if empty
    const float mc = m_new * cl;
    u32x4_t pf[2];
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = fast_exp2(fmaf(sc[r], cl, -mc)), p1 = fast_exp2(fmaf(sc[r + 1], cl, -mc));
      rs += p0 + p1;
      pf[r >> 3][(r & 7) >> 1] = pack_bf16(p0, p1);
    }
    l = l * alpha + rs;
    m = m_new;
#pragma unroll
    for (int d = 0; d < T::DB; ++d) acc[d] *= alpha;

    // V^T tile of this wave, keys permuted to the score register order
    wave_lds_order();
#pragma unroll
    for (int g = 0; g < T::NG; ++g) {
      const int pos = vt_pos16(4 * vq);
      const int dcol = 8 * (vcol0 + (T::CPR / T::NG) * g);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x0 = vr[buf][g][0][w], x1 = vr[buf][g][1][w], x2 = vr[buf][g][2][w],
                       x3 = vr[buf][g][3][w];
        uint16_t* even = vt + (dcol + 2 * w) * T::VT_LD + pos;
        *reinterpret_cast<u32x2_t*>(even) =
            u32x2_t{(x0 & 0xffffu) | (x1 << 16), (x2 & 0xffffu) | (x3 << 16)};
        *reinterpret_cast<u32x2_t*>(even + T::VT_LD) =
            u32x2_t{(x0 >> 16) | (x1 & 0xffff0000u), (x2 >> 16) | (x3 & 0xffff0000u)};
      }
    }
    wave_lds_order();
#pragma unroll
    for (int d = 0; d < T::DB; ++d)
#pragma unroll
      for (int ts = 0; ts < 2; ++ts) {
        const u32x4_t a =
            *reinterpret_cast<const u32x4_t*>(vt + (32 * d + l32) * T::VT_LD + 16 * ts + 8 * hi);
        acc[d] = mfma32(a, pf[ts], acc[d]);
      }
    wave_lds_order();
  };

  // Software pipeline: the wave's next block is in flight while the current one
  // computes.  Loads are unconditional (a block past the chunk has a zero-length
  // descriptor and reads zeros without touching memory) and the trip count is rounded
  // up to even; a trailing empty step leaves (m, l, acc) unchanged since every score
  // is -inf.  Waves without a block skip the loop.
  const int mine = wave < nb ? (nb - wave + kDecWaves - 1) / kDecWaves : 0;
  if (mine > 0) {
    load(0, wave);
    for (int n = 0; n < mine; n += 2) {
      const int b0 = wave + kDecWaves * n;
      load(1, b0 + kDecWaves);
      step(0, b0);
      load(0, b0 + 2 * kDecWaves);
      step(1, b0 + kDecWaves);
    }
  }
  l = halves_sum(l);

  // ---- merge the four waves' partial states
  __syncthreads();
  float* mrg = reinterpret_cast<float*>(lds);
  if (wave > 0) {
    float* r = mrg + (wave - 1) * T::MRG_FLOATS;
    if (hi == 0) {
      r[l32] = m;
      r[32 + l32] = l;
    }
#pragma unroll
    for (int d = 0; d < T::DB; ++d)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr)
        r[64 + (32 * d + 8 * (rr >> 2) + 4 * hi + (rr & 3)) * 32 + l32] = acc[d][rr];
  }
  __syncthreads();
  if (wave != 0) return;
  float M = m;
#pragma unroll
  for (int w = 0; w < kDecWaves - 1; ++w) M = fmaxf(M, mrg[w * T::MRG_FLOATS + l32]);
  const float a0 = fast_exp2((m - M) * cl);  // wave 0 always holds block 0: M, m finite
  float lt = l * a0;
#pragma unroll
  for (int d = 0; d < T::DB; ++d) acc[d] *= a0;
#pragma unroll
  for (int w = 0; w < kDecWaves - 1; ++w) {
    const float* r = mrg + w * T::MRG_FLOATS;
    const float aw = fast_exp2((r[l32] - M) * cl);  // 0 for a wave that had no block
    lt += r[32 + l32] * aw;
#pragma unroll
    for (int d = 0; d < T::DB; ++d)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr)
        acc[d][rr] += aw * r[64 + (32 * d + 8 * (rr >> 2) + 4 * hi + (rr & 3)) * 32 + l32];
  }
  if (!hvalid) return;
  const float inv = 1.f / lt;
  const int64_t row = ((int64_t)s * p.Hq + hq) * p.nsplit + c;
  float* po = p.part_o + row * D;
#pragma unroll
  for (int d = 0; d < T::DB; ++d)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg)
      *reinterpret_cast<f32x4_t*>(po + 32 * d + 8 * rg + 4 * hi) =
          f32x4_t{acc[d][4 * rg] * inv, acc[d][4 * rg + 1] * inv, acc[d][4 * rg + 2] * inv,
                  acc[d][4 * rg + 3] * inv};
  if (hi == 0) p.part_lse[row] = M * p.scale + __logf(lt);
}

// One workgroup of 64 lanes per (sequence, query head): merge the chunk partials.
template <int D, bool OUT_F32>
__global__ void __launch_bounds__(64) decode_merge_kernel(DecParams p) {
  const int s = blockIdx.x / p.Hq, hq = blockIdx.x % p.Hq;
  const int tid = threadIdx.x;
  int L = p.seq_lens[s];
  L = L < 0 ? 0 : (L > p.max_len ? p.max_len : L);
  const int n = (L + p.split_len - 1) / p.split_len;
  const int64_t row0 = ((int64_t)s * p.Hq + hq) * p.nsplit;
  const float* pl = p.part_lse + row0;
  float M = -INFINITY;
  for (int c = 0; c < n; ++c) M = fmaxf(M, pl[c]);
  constexpr int E = D / 64;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float tot = 0.f;
  for (int c = 0; c < n; ++c) {
    const float w = fast_exp2((pl[c] - M) * kLog2e);
    tot += w;
    const float* po = p.part_o + (row0 + c) * D;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = fmaf(w, po[tid + 64 * e], acc[e]);
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
  if constexpr (OUT_F32) {
    float* o = static_cast<float*>(p.o) + s * p.os0 + (int64_t)hq * p.os1;
#pragma unroll
    for (int e = 0; e < E; ++e) o[tid + 64 * e] = acc[e] * inv;
  } else {
    uint16_t* o = static_cast<uint16_t*>(p.o) + s * p.os0 + (int64_t)hq * p.os1;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint32_t pk = pack_bf16(acc[e] * inv, 0.f);
      o[tid + 64 * e] = static_cast<uint16_t>(pk & 0xffffu);
    }
  }
  if (p.lse && tid == 0) p.lse[(int64_t)s * p.Hq + hq] = tot > 0.f ? M + __logf(tot) : -INFINITY;
}

template <typename K>
hipError_t launch(K kernel, dim3 grid, dim3 block, const DecParams& p, hipStream_t stream) {
  DecParams local = p;
  void* args[] = {&local};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0, stream);
}

}  // namespace

size_t decode_workspace_bytes(int Bs, int Hq, int nsplit, int D) {
  const size_t rows = (size_t)Bs * Hq * nsplit;
  const size_t o_bytes = (rows * D * 4 + 255) & ~size_t(255);
  return o_bytes + ((rows * 4 + 255) & ~size_t(255));
}

hipError_t launch_decode(const DecParams& p, int D, int out_dtype, hipStream_t stream) {
  if (p.nsplit > 0) {
    const dim3 grid(p.nsplit, p.Hkv * p.nhb, p.Bs);
    const hipError_t e = D == 128 ? launch(decode_split_kernel<128>, grid, dim3(256), p, stream)
                                  : launch(decode_split_kernel<64>, grid, dim3(256), p, stream);
    if (e != hipSuccess) return e;
  }
  const dim3 mgrid(p.Bs * p.Hq);
  const bool f32 = out_dtype == FA_F32;
  if (D == 128)
    return f32 ? launch(decode_merge_kernel<128, true>, mgrid, dim3(64), p, stream)
               : launch(decode_merge_kernel<128, false>, mgrid, dim3(64), p, stream);
  return f32 ? launch(decode_merge_kernel<64, true>, mgrid, dim3(64), p, stream)
             : launch(decode_merge_kernel<64, false>, mgrid, dim3(64), p, stream);
}

}  // namespace fa
