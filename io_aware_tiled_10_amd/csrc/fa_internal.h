// fa_internal.h -- kernel parameter blocks and launchers behind the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Forward.  Strides are in elements; the dim dimension is contiguous.
struct FwdParams {
  const uint16_t* q;  // bf16 bits (or fp32 reinterpreted by the fp32 kernel)
  const uint16_t* k;
  const uint16_t* v;
  void* o;
  float* lse;
  const int32_t* kv_lens;
  // packed variable-length batch: sequence b owns rows cu_q[b] .. cu_q[b+1] of q / o
  // and cu_k[b] .. cu_k[b+1] of k / v (batch strides unused); NULL for [B, H, N, D]
  const int32_t* cu_q;
  const int32_t* cu_k;
  int total_q, total_k;
  int64_t qs0, qs1, qs2, ks0, ks1, ks2, vs0, vs1, vs2, os0, os1, os2;
  int64_t lse_sb, lse_sh;  // LSE element of (b, h, row): b * lse_sb + h * lse_sh + row
  // FP8 Q K^T: q and k hold E4M3 codes (strides in bytes); the step of each 64-row block
  // is q_scale[b * qsc_b + h * qsc_h + row / 64] (k_scale likewise, per KV head)
  const float* q_scale;
  const float* k_scale;
  int64_t qsc_b, qsc_h, ksc_b, ksc_h;
  // dropout on P (when drop_t > 0): keep iff the Philox byte >= drop_t, scale kept values
  // by drop_scale = 256 / (256 - drop_t)
  uint32_t drop_t, seed_lo, seed_hi;
  float drop_scale;
  int B, Hq, Hkv, Nq, Nk, G, nqt;  // packed batches: Nq = longest sequence
  int th;  // bf16 forward: query heads of one GQA group that share a workgroup tile
  int gsz; // bf16 forward: (batch entry, KV head) groups an XCD takes at a time
  float scale, scale_log2;
  int causal;
};

hipError_t launch_fwd(const FwdParams& p, int in_dtype, int out_dtype, int D, hipStream_t stream);
// bf16 forward with dropout on P (p.drop_t > 0, p.seed_*, p.drop_scale).
hipError_t launch_fwd_dropout(const FwdParams& p, int out_dtype, int D, hipStream_t stream);
// Q and K as E4M3 codes with per-64-row steps, V bf16 (D = 128).
hipError_t launch_fwd_fp8(const FwdParams& p, int out_dtype, hipStream_t stream);

// E4M3 block quantisation of a bf16 [B, H, N, D] tensor.
struct QuantParams {
  const uint16_t* x;
  uint8_t* codes;
  float* scales;  // contiguous [B, H, nb]
  int64_t xs0, xs1, xs2, cs0, cs1, cs2;
  int B, H, N, nb;
};
hipError_t launch_quantize_fp8(const QuantParams& p, int D, hipStream_t stream);

// Backward.
struct BwdParams {
  const uint16_t *q, *k, *v, *o, *dout;
  const float* lse;
  uint16_t *dq, *dk, *dv;
  const int32_t* kv_lens;
  float* lse2;    // [B, Hq, Nq] workspace: LSE * log2 e of each query row (+inf if LSE = -inf)
  float* negd;    // [B, Hq, Nq] workspace: -D_i = -sum_d dO_id O_id of each query row
  int64_t qs0, qs1, qs2, ks0, ks1, ks2, vs0, vs1, vs2, os0, os1, os2, dos0, dos1, dos2;
  int64_t dqs0, dqs1, dqs2, dks0, dks1, dks2, dvs0, dvs1, dvs2;
  int B, Hq, Hkv, Nq, Nk, G, nkt;
  int gsz;  // (batch entry, KV head) groups an XCD takes at a time, per kernel
  float scale, scale_log2;
  int causal;
  uint32_t drop_t, seed_lo, seed_hi;  // dropout as in the forward (drop_t == 0: none)
  float drop_scale;
};

size_t bwd_workspace_bytes(int B, int Hq, int Nq, int D);
// Points p.lse2 and p.negd into a workspace of bwd_workspace_bytes() bytes (p.B, p.Hq
// and p.Nq set).
void bwd_bind_workspace(BwdParams& p, void* workspace, int D);
hipError_t launch_bwd(const BwdParams& p, int D, hipStream_t stream);

// Split-KV decode.
struct DecParams {
  const uint16_t* q;
  const uint16_t *k, *v;
  const int32_t* seq_lens;
  void* o;
  float* lse;
  float* part_o;    // [Bs, Hq, nsplit, D]
  float* part_lse;  // [Bs, Hq, nsplit]
  int64_t qs0, qs1, ks0, ks1, ks2, vs0, vs1, vs2, os0, os1;
  int Bs, Hq, Hkv, G, nhb, max_len, split_len, nsplit;
  float scale, scale_log2;
  // paged cache (NULL table: contiguous [Bs, Hkv, cache_len, D]): k / v point at the
  // page pool, ks0 / vs0 are page strides, position t of sequence s is row
  // t % 2^page_shift of page table[s * table_stride + (t >> page_shift)]
  const int32_t* table;
  int64_t table_stride;
  int page_shift, num_pages;
};

size_t decode_workspace_bytes(int Bs, int Hq, int nsplit, int D);
hipError_t launch_decode(const DecParams& p, int D, int out_dtype, hipStream_t stream);

// The static per-device array that fa_decode_noalloc uses as its workspace, and its
// address on the current device (looked up once per device, then cached).
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
hipError_t decode_scratch(void** ptr);

}  // namespace fa
