// fa_quant.hip -- E4M3 block quantisation of Q or K for the FP8 forward, for gfx950.
//
// Method (V2/V3 article, aiqz.cc, section FP8低精度 and its formula block): pass 1
// finds max|x| over a block and sets the step Delta = max|x| / 448 (448 is the largest
// E4M3 value); pass 2 stores x / Delta rounded to E4M3.  A block is 64 rows of one
// head (all D columns); an all-zero block gets Delta = 1.  Both divisions are single
// correctly rounded fp32 divisions, and the conversion is the hardware's round to
// nearest even into OCP E4M3 (after clamping to +-448, since out-of-range inputs would
// convert to NaN).
//
// gfx950 mapping: one workgroup of 256 lanes per (batch, head, block); each lane owns
// 32 consecutive elements of one row, keeps them in registers between the two passes,
// and writes its 32 codes with two 16-byte stores.  The block maximum is a wave
// reduction followed by an LDS exchange between the four waves.
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kQuantRows = 64;

template <int D>
__global__ void __launch_bounds__(256) quant_fp8_kernel(QuantParams p) {
  constexpr int LPR = D / 32;                    // lanes per row
  static_assert(kQuantRows * LPR == 256, "one workgroup covers one block");
  __shared__ float wmax[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int blk = blockIdx.x % p.nb, bh = blockIdx.x / p.nb;
  const int h = bh % p.H, b = bh / p.H;
  const int row = blk * kQuantRows + tid / LPR, col = 32 * (tid % LPR);
  const bool valid = row < p.N;

  float x[32];
  if (valid) {
    const uint16_t* src = p.x + b * p.xs0 + h * p.xs1 + (int64_t)row * p.xs2 + col;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const u32x4_t w = *reinterpret_cast<const u32x4_t*>(src + 8 * v);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[8 * v + 2 * e] = bf16_lo(w[e]);
        x[8 * v + 2 * e + 1] = bf16_hi(w[e]);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 32; ++e) x[e] = 0.f;
  }
  // pass 1: max |x| over the block
  float a = 0.f;
#pragma unroll
  for (int e = 0; e < 32; ++e) a = fmaxf(a, fabsf(x[e]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
  if (lane == 0) wmax[wave] = a;
  __syncthreads();
  a = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float delta = a > 0.f ? __fdiv_rn(a, 448.f) : 1.f;
  if (tid == 0) p.scales[(int64_t)bh * p.nb + blk] = delta;
  if (!valid) return;
  // pass 2: codes of x / Delta
  uint32_t c[8];
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = fminf(fmaxf(__fdiv_rn(x[4 * w + e], delta), -448.f), 448.f);
    uint32_t pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    pk = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], pk, true);
    c[w] = pk;
  }
  uint8_t* dst = p.codes + b * p.cs0 + h * p.cs1 + (int64_t)row * p.cs2 + col;
  *reinterpret_cast<u32x4_t*>(dst) = u32x4_t{c[0], c[1], c[2], c[3]};
  *reinterpret_cast<u32x4_t*>(dst + 16) = u32x4_t{c[4], c[5], c[6], c[7]};
}

}  // namespace

hipError_t launch_quantize_fp8(const QuantParams& p, int D, hipStream_t stream) {
  const int64_t grid = (int64_t)p.B * p.H * p.nb;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  QuantParams local = p;
  void* args[] = {&local};
  if (D != 128) return hipErrorInvalidValue;
  return hipLaunchKernel(reinterpret_cast<const void*>(quant_fp8_kernel<128>), dim3((unsigned)grid),
                         dim3(256), args, 0, stream);
}

}  // namespace fa
