// fa_common.h -- device helpers shared by the gfx950 attention kernels.
//
// Vector types, the bf16 MFMA used for both attention contractions, bf16 packing,
// cross-half-wave exchange, and the XCD-aware workgroup order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa.h"

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, each with its own L2

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16) on the matrix cores.
// Operand layout (wave64): lane l supplies row (A) / column (B) l % 32 and eight
// consecutive k-elements of half l / 32.  Result: lane l holds column l % 32, and
// register r holds row 8*(r/4) + 4*(l/32) + r%4.
__device__ __forceinline__ f32x16_t mfma32(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
// 32x32x64 MFMA on OCP E4M3 operands (format code 0 for both), unscaled, fp32
// accumulate.  Lane l holds row (A) / column (B) l % 32 and 32 bytes of the k range;
// byte b of lane half h in A multiplies byte b of the same half in B, so any
// assignment of k to (half, byte) works as long as both operands use the same one.
// The result registers are laid out as those of the bf16 32x32x16 product.
__device__ __forceinline__ f32x16_t mfma32_f8(i32x8_t a, i32x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ i32x8_t cat8(u32x4_t a, u32x4_t b) {
  return __builtin_bit_cast(i32x8_t, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Two floats -> packed bf16 pair (round to nearest even); `lo` in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v = (bf16x2_t){(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// max / sum of the values held by lanes l and l ^ 32.  The swap returns the lane's own
// value and the other half's value as its two results; a symmetric combine of both
// does not depend on which result is which.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup order: the dispatcher hands consecutive workgroup ids to the 8 XCDs in
// turn.  Remap so that each XCD receives one contiguous range of logical tiles
// (tiles that share K/V then share that XCD's L2).  A bijection on [0, total).
__device__ __forceinline__ int xcd_contiguous(int id, int total) {
  const int x = id % kNumXcd, k = id / kNumXcd;
  const int q = total / kNumXcd, r = total % kNumXcd;
  return x * q + (x < r ? x : r) + k;
}

// Tile order for a grid of npair groups (batch entry, KV head) x nrank ranks x ng heads
// (total = npair * nrank * ng).  Each XCD receives a contiguous range of whole groups, so
// the tiles that share a group's K/V share that XCD's L2.  When the groups split evenly
// over the XCDs, each XCD takes its groups gsz at a time (all of them when gsz <= 0), and
// inside such a batch of groups the rank varies slowest: the rank-0 tiles of the batch
// first, then rank 1, ..., which with rank 0 the heaviest gives a longest-first schedule.
// A small gsz keeps few groups' K/V in flight on an XCD at once (gsz = 1: one group's
// tiles after another's), so that they stay in its L2.  Otherwise (or without
// rank_major) ranks vary right after the heads.
struct TileId {
  int gi, rank, pair;
};
__device__ __forceinline__ TileId tile_order(int id, int total, int npair, int nrank, int ng,
                                             bool rank_major = true, int gsz = 0) {
  const int t = xcd_contiguous(id, total);
  TileId r;
  if (rank_major && npair % kNumXcd == 0) {
    const int per = npair / kNumXcd, span = per * nrank * ng;
    const int x = t / span;
    int u = t - x * span;
    r.gi = u % ng;
    u /= ng;
    // groups of gsz consecutive pairs (the last one may be smaller), one after another;
    // rank-major inside each group
    const int gs = (gsz <= 0 || gsz > per) ? per : gsz;
    const int g = u / (gs * nrank), w = u - g * gs * nrank;
    const int gl = min(gs, per - g * gs);
    r.rank = w / gl;
    r.pair = x * per + g * gs + w % gl;
  } else {
    r.gi = t % ng;
    const int u = t / ng;
    r.rank = u % nrank;
    r.pair = u / nrank;
  }
  return r;
}

__device__ __forceinline__ const uint16_t* as_u16(const void* p) {
  return static_cast<const uint16_t*>(p);
}

// Raw buffer resource over [base, base + bytes): a 16-byte load whose offset lies past
// the end returns zeros, so rows beyond a valid length need no branch and no select.
// 0x00020000 is the gfx9-family third descriptor word for untyped 32-bit data.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
// The same load marked non-temporal (cache policy bit "nt"): for data read exactly once,
// such as a KV cache streamed by the decode, so it does not displace reused lines.
__device__ __forceinline__ u32x4_t buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2));
}

// Direct global -> LDS load (gfx950 LDS DMA): lane t's 16 bytes, read at byte `off` of
// the buffer, land at lds + 16 t; the register file is bypassed.  Out-of-range bytes are
// written as zeros.  `lds` must be the same for the whole wave.  The compiler does not
// track these writes: the issuing code waits with wait_vmcnt before reading them.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t off,
                                          int aux = 0, int soff = 0) {
  if (aux)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                             (int)off, soff, 0, 2);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                             (int)off, soff, 0, 0);
}

// The same with 4 bytes per lane: lane t's dword lands at lds + 4 t (256 bytes per wave).
__device__ __forceinline__ void lds_dma4(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, (int)off, 0, 0, 0);
}

// Wait until at most N vector-memory operations of this wave are outstanding; also a
// compiler barrier for memory accesses.
//
// FA_DEBUG_SYNC builds (a race canary): every counted wait waits for all of the wave's
// outstanding operations, and every fence-free barrier first drains the wave's loads and
// LDS reads.  The arithmetic is unchanged, so such a build must give the same bits; a
// wait count that were too loose would show up as a difference.
#ifdef FA_DEBUG_SYNC
#define FA_WAIT_VMCNT(N) asm volatile("s_waitcnt vmcnt(0)" ::: "memory")
#else
#define FA_WAIT_VMCNT(N) asm volatile("s_waitcnt vmcnt(" #N ")" ::: "memory")
#endif
#define FA_WAIT_LGKMCNT0() asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory")
// FA_WAIT_VMCNT for a compile-time count (the counts the ring pipelines use).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N == 0 || N == 1 || N == 2 || N == 3 || N == 4 || N == 5 || N == 8 || N == 9 ||
                    N == 16,
                "add the count here");
  if constexpr (N == 0) FA_WAIT_VMCNT(0);
  else if constexpr (N == 1) FA_WAIT_VMCNT(1);
  else if constexpr (N == 2) FA_WAIT_VMCNT(2);
  else if constexpr (N == 3) FA_WAIT_VMCNT(3);
  else if constexpr (N == 4) FA_WAIT_VMCNT(4);
  else if constexpr (N == 5) FA_WAIT_VMCNT(5);
  else if constexpr (N == 8) FA_WAIT_VMCNT(8);
  else if constexpr (N == 9) FA_WAIT_VMCNT(9);
  else FA_WAIT_VMCNT(16);
}
// Philox4x32 with 10 rounds (Salmon, Moraes, Dror and Shaw, "Parallel random numbers:
// as easy as 1, 2, 3", SC 2011): four 32-bit words from a 4-word counter and a 2-word key.
__device__ __forceinline__ u32x4_t philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    // each 32 x 32 -> 64-bit product is one v_mad_u64_u32 (high and low words at once)
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    c0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    c1 = (uint32_t)p1;
    c2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c3 = (uint32_t)p0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return u32x4_t{c0, c1, c2, c3};
}

// Dropout mask words of one query row and one group of 16 keys: the keys
// 32 c + 4 h2 + 8 a + e (a, e = 0..3) of query i, head h, batch entry b take byte 4 a + e
// of philox(2 c + h2, i, h, b; seed).  Byte n sits at bits 8 (n % 4) of word n / 4.
__device__ __forceinline__ u32x4_t dropout_words(int chunk, int h2, int i, int h, int b,
                                                 uint32_t seed_lo, uint32_t seed_hi) {
  return philox4x32_10((uint32_t)(2 * chunk + h2), (uint32_t)i, (uint32_t)h, (uint32_t)b, seed_lo, seed_hi);
}
__device__ __forceinline__ bool dropout_keep(uint32_t word, int byte, uint32_t threshold) {
  return ((word >> (8 * byte)) & 0xffu) >= threshold;
}

// Workgroup barrier without the memory fence __syncthreads() adds (which waits for every
// outstanding load, ring prefetches included).  Callers order LDS themselves: each wave
// waits for its own ring loads (FA_WAIT_VMCNT) and LDS reads (lgkmcnt) before it.
#ifdef FA_DEBUG_SYNC
#define FA_BARRIER() asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory")
#else
#define FA_BARRIER() asm volatile("s_barrier" ::: "memory")
#endif

// gfx950 transposing LDS read (ds_read_b64_tr_b16) of 4 bf16 values per lane.  Within
// each group of 16 lanes, let M be the 16 x 4 matrix whose row i is the 8 bytes at lane
// i's address; lane j receives M[j/4 + 4e][j%4] for e = 0..3, packed two per dword.
// Issued from inline assembly so that the compiler neither waits for unrelated LDS-DMA
// loads before it nor tracks its completion: the caller must run lds_wait_tr on the
// results before using them.  Two reads at byte offsets O0 and O1 from `addr`.
template <int O0, int O1>
__device__ __forceinline__ void lds_read_tr16x2(u32x2_t& a, u32x2_t& b, uint32_t addr) {
  asm volatile("ds_read_b64_tr_b16 %0, %2 offset:%3\n\tds_read_b64_tr_b16 %1, %2 offset:%4"
               : "=&v"(a), "=&v"(b)
               : "v"(addr), "i"(O0), "i"(O1)
               : "memory");
}
template <int O0>
__device__ __forceinline__ void lds_read_tr16(u32x2_t& a, uint32_t addr) {
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(a) : "v"(addr), "i"(O0) : "memory");
}
__device__ __forceinline__ void lds_wait_tr2(u32x2_t& a, u32x2_t& b) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b)::"memory");
}
// Wait for all outstanding LDS reads of this wave; the operands tie the results of
// earlier lds_read_tr16x2 calls to this point, so no use of them moves above the wait.
__device__ __forceinline__ void lds_wait_tr(u32x2_t& a, u32x2_t& b, u32x2_t& c, u32x2_t& d) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d)::"memory");
}
// The same with at most N LDS operations of this wave still outstanding (LDS results
// return in issue order, so the reads issued more than N operations ago have landed).
template <int N>
__device__ __forceinline__ void lds_wait_tr(u32x2_t& a, u32x2_t& b, u32x2_t& c, u32x2_t& d) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt holds 0..15");
#ifdef FA_DEBUG_SYNC
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d)::"memory");
#else
  asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d) : "i"(N) : "memory");
#endif
}
// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Bytes a buffer over `rows` rows of `pitch_bytes` must span so that every 16-byte
// chunk of each of those rows (width row_bytes) is in range and the next row is not.
__device__ __forceinline__ uint32_t rows_span(int rows, int64_t pitch_bytes, int row_bytes) {
  return rows <= 0 ? 0u : (uint32_t)((int64_t)(rows - 1) * pitch_bytes + row_bytes);
}

}  // namespace fa
