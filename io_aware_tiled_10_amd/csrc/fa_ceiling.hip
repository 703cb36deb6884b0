// fa_ceiling.hip -- measurement aids: the sustained rate of the bf16 matrix cores on this
// part with operands of a given bit pattern and no memory traffic at all, and the HBM read
// rate of a plain streaming kernel.
//
// The attention kernels are priced against the published dense bf16 peak.  How much of
// that peak the chip sustains depends on the data the matrix cores multiply (their power
// draw, and so the clock they hold, grows with operand bit activity).  This kernel runs
// nothing but 32x32x16 bf16 MFMAs, in the forward's occupancy (8 waves per workgroup,
// two per SIMD), on operands held in registers: the upper bound any kernel on data of
// that kind can reach.  Each wave holds 8 A and 8 B fragments and cycles through them,
// so consecutive products never see the same pair of operands, into four independent
// accumulator chains.
#include "fa_ceiling.h"
#include "fa_common.h"

namespace fa {
namespace {

constexpr int kWaves = 8;
constexpr int kFrags = 8;

// 32-bit mixing function (the finaliser of the 32-bit MurmurHash3)
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x85ebca6bu;
  x ^= x >> 13;
  x *= 0xc2b2ae35u;
  x ^= x >> 16;
  return x;
}

// pattern 0: bf16 values of random sign, exponent in [2^-2, 2^2) and random mantissa
// (the spread of N(0,1) data); pattern 1: every value 1.0
__device__ __forceinline__ uint32_t operand_word(int pattern, uint32_t seed) {
  if (pattern == 1) return 0x3f803f80u;
  const uint32_t r = mix32(seed);
  auto half = [](uint32_t b) {  // sign | exponent 125..128 | 7 mantissa bits
    return (uint32_t)((b & 0x8000u) | ((125u + ((b >> 7) & 3u)) << 7) | (b & 0x7fu));
  };
  return half(r & 0xffffu) | (half(r >> 16) << 16);
}

__global__ void __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2)))
mfma_ceiling_kernel(float* out, int iters, int pattern) {
  const uint32_t tid = blockIdx.x * blockDim.x + threadIdx.x;
  u32x4_t a[kFrags], b[kFrags];
#pragma unroll
  for (int f = 0; f < kFrags; ++f)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      a[f][w] = operand_word(pattern, tid * 64u + (uint32_t)(f * 8 + w));
      b[f][w] = operand_word(pattern, tid * 64u + (uint32_t)(f * 8 + 4 + w) + 0x9e3779b9u);
    }
  f32x16_t acc[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int f = 0; f < kFrags; ++f) acc[f & 3] = mfma32(a[f], b[(f + 3) & (kFrags - 1)], acc[f & 3]);
#pragma unroll
    for (int f = 0; f < kFrags; ++f) acc[f & 3] = mfma32(a[(f + 5) & (kFrags - 1)], b[f], acc[f & 3]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[tid] = s;  // keeps every product live
}

constexpr int kStreamThreads = 256, kStreamInFlight = 8;

// HBM streaming read: workgroup g reads its contiguous slice of `per` 16-byte elements with
// non-temporal loads, kStreamInFlight of them in flight per thread, and stores one word per
// thread (the XOR of what it read, so that no load is dropped).
__global__ void __launch_bounds__(kStreamThreads) stream_read_kernel(const u32x4_t* src, int64_t per,
                                                                     uint32_t* out) {
  const u32x4_t* p = src + (int64_t)blockIdx.x * per;
  uint32_t acc = 0;
  for (int64_t i = threadIdx.x; i < per; i += kStreamThreads * kStreamInFlight) {
    u32x4_t v[kStreamInFlight];
#pragma unroll
    for (int u = 0; u < kStreamInFlight; ++u) v[u] = __builtin_nontemporal_load(p + i + kStreamThreads * u);
#pragma unroll
    for (int u = 0; u < kStreamInFlight; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  out[blockIdx.x * kStreamThreads + threadIdx.x] = acc;
}

}  // namespace
}  // namespace fa

extern "C" int fa_ceiling_stream(const void* src, int64_t bytes, unsigned int* out, int workgroups,
                                 void* stream) {
  const int64_t chunk = (int64_t)16 * fa::kStreamThreads * fa::kStreamInFlight;  // one trip of a workgroup
  if (!src || !out || workgroups < 1 || bytes <= 0 || bytes % (chunk * workgroups) != 0) return 1;
  if (reinterpret_cast<uintptr_t>(src) & 15u) return 1;
  const fa::u32x4_t* s = static_cast<const fa::u32x4_t*>(src);
  int64_t per = bytes / 16 / workgroups;
  uint32_t* o = out;
  void* args[] = {&s, &per, &o};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(fa::stream_read_kernel),
                                       dim3((unsigned)workgroups), dim3(fa::kStreamThreads), args, 0,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? 0 : 2;
}

extern "C" int fa_ceiling_mfma(float* out, int workgroups, int iters, int pattern, void* stream) {
  if (!out || workgroups < 1 || iters < 1 || (pattern != 0 && pattern != 1)) return 1;
  void* args[] = {&out, &iters, &pattern};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(fa::mfma_ceiling_kernel),
                                       dim3((unsigned)workgroups), dim3(64 * fa::kWaves), args, 0,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? 0 : 2;
}

extern "C" double fa_ceiling_mfma_flops(int workgroups, int iters) {
  // 16 products per trip, 2 * 32 * 32 * 16 FLOP each, per wave
  return (double)workgroups * fa::kWaves * iters * 16.0 * 2.0 * 32 * 32 * 16;
}
