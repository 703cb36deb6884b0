// fa_api.cpp -- the extern "C" entry points of libfa.so: argument validation on the
// host, then kernel launches on the caller's stream.  Validation makes no HIP call,
// so every rejection path is exercised without a GPU.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "fa.h"
#include "fa_internal.h"

static_assert(fa::kDecodeScratchBytes == FA_DECODE_NOALLOC_MAX_WORKSPACE_BYTES,
              "the header states the decode scratch size");

namespace fa {

// Backward workspace: two fp32 planes over the query rows, LSE * log2 e and then -D_i,
// each rounded up to 256 bytes.
static size_t bwd_plane_bytes(int B, int Hq, int Nq) { return ((size_t)B * Hq * Nq * 4 + 255) & ~size_t(255); }

size_t bwd_workspace_bytes(int B, int Hq, int Nq, int D) {
  (void)D;
  return 2 * bwd_plane_bytes(B, Hq, Nq);
}

void bwd_bind_workspace(BwdParams& p, void* workspace, int D) {
  (void)D;
  p.lse2 = static_cast<float*>(workspace);
  p.negd = reinterpret_cast<float*>(static_cast<char*>(workspace) + bwd_plane_bytes(p.B, p.Hq, p.Nq));
}

// Decode workspace: partial O [Bs, Hq, nsplit, D] fp32, then partial LSE [Bs, Hq, nsplit]
// fp32, each rounded up to 256 bytes.
size_t decode_workspace_bytes(int Bs, int Hq, int nsplit, int D) {
  const size_t rows = (size_t)Bs * Hq * nsplit;
  const size_t o_bytes = (rows * D * 4 + 255) & ~size_t(255);
  return o_bytes + ((rows * 4 + 255) & ~size_t(255));
}

}  // namespace fa

namespace {

constexpr int kMaxHeads = 1 << 16;
constexpr int kMaxGridYZ = 65535;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool strides_ok(const int64_t* st, int n, int elem_bytes) {
  for (int i = 0; i < n; ++i) {
    if (st[i] < 0) return false;
    if ((st[i] * elem_bytes) % 16 != 0) return false;
  }
  return true;
}

bool scale_ok(float s) { return std::isfinite(s) && s > 0.f; }

// Row-to-row strides reach the kernels' 32-bit buffer offsets multiplied by up to 256
// rows; 8 MiB per row keeps every such offset below 2^31.
constexpr int64_t kMaxPitchBytes = int64_t(1) << 23;
bool pitch_ok(int64_t stride_elems, int elem_bytes) { return stride_elems * elem_bytes <= kMaxPitchBytes; }

fa_status map_launch_error(hipError_t e) {
  switch (e) {
    case hipSuccess:
      return FA_OK;
    case hipErrorNoDevice:
    case hipErrorInvalidDevice:
    case hipErrorNoBinaryForGpu:
    case hipErrorInvalidDeviceFunction:
    case hipErrorInsufficientDriver:
      return FA_ERR_DEVICE;
    default:
      return FA_ERR_LAUNCH;
  }
}

fa_status validate_fwd(const fa_fwd_args* a) {
  if (!a) return FA_ERR_NULL_PTR;
  if (a->B < 1 || a->Hq < 1 || a->Hkv < 1 || a->Nq < 0 || a->Nk < 0 || a->D < 1)
    return FA_ERR_SHAPE;
  if (a->Hq > kMaxHeads || a->Hkv > a->Hq || a->Hq % a->Hkv != 0) return FA_ERR_SHAPE;
  if (a->in_dtype != FA_BF16 && a->in_dtype != FA_F32) return FA_ERR_DTYPE;
  if (a->out_dtype != FA_BF16 && a->out_dtype != FA_F32) return FA_ERR_DTYPE;
  if (a->in_dtype == FA_F32 && a->out_dtype != FA_F32) return FA_ERR_DTYPE;
  if (a->in_dtype == FA_BF16 && a->D != 64 && a->D != 128) return FA_ERR_UNSUPPORTED;
  if (a->in_dtype == FA_F32 && a->D != 64) return FA_ERR_UNSUPPORTED;
  if (!scale_ok(a->scale)) return FA_ERR_ARG;
  if (a->causal != 0 && a->causal != 1) return FA_ERR_ARG;
  if (a->Nq == 0) return FA_OK;
  if (!a->q || !a->o) return FA_ERR_NULL_PTR;
  if (a->Nk > 0 && (!a->k || !a->v)) return FA_ERR_NULL_PTR;  // never read when Nk == 0
  const int ib = a->in_dtype == FA_BF16 ? 2 : 4, ob = a->out_dtype == FA_BF16 ? 2 : 4;
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o))
    return FA_ERR_STRIDE;
  if (!strides_ok(a->q_stride, 3, ib) || !strides_ok(a->k_stride, 3, ib) ||
      !strides_ok(a->v_stride, 3, ib) || !strides_ok(a->o_stride, 3, ob))
    return FA_ERR_STRIDE;
  if (!pitch_ok(a->q_stride[2], ib) || !pitch_ok(a->k_stride[2], ib) || !pitch_ok(a->v_stride[2], ib))
    return FA_ERR_SHAPE;
  if (a->lse && (reinterpret_cast<uintptr_t>(a->lse) & 3u)) return FA_ERR_STRIDE;
  return FA_OK;
}

fa_status validate_bwd(const fa_bwd_args* a) {
  if (!a) return FA_ERR_NULL_PTR;
  if (a->B < 1 || a->Hq < 1 || a->Hkv < 1 || a->Nq < 0 || a->Nk < 0 || a->D < 1)
    return FA_ERR_SHAPE;
  if (a->Hq > kMaxHeads || a->Hkv > a->Hq || a->Hq % a->Hkv != 0) return FA_ERR_SHAPE;
  if (a->dtype != FA_BF16) return FA_ERR_DTYPE;
  if (a->D != 64 && a->D != 128) return FA_ERR_UNSUPPORTED;
  if (!scale_ok(a->scale)) return FA_ERR_ARG;
  if (a->causal != 0 && a->causal != 1) return FA_ERR_ARG;
  if (a->Nk > 0 && (!a->k || !a->v || !a->dk || !a->dv)) return FA_ERR_NULL_PTR;
  if (a->Nq > 0 && (!a->q || !a->o || !a->dout || !a->lse || !a->dq)) return FA_ERR_NULL_PTR;
  const void* ptrs[] = {a->q, a->k, a->v, a->o, a->dout, a->dq, a->dk, a->dv};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FA_ERR_STRIDE;
  const int64_t* st[] = {a->q_stride,  a->k_stride,  a->v_stride,  a->o_stride,
                         a->do_stride, a->dq_stride, a->dk_stride, a->dv_stride};
  for (const int64_t* s : st)
    if (!strides_ok(s, 3, 2)) return FA_ERR_STRIDE;
  for (const int64_t* s : st)
    if (!pitch_ok(s[2], 2)) return FA_ERR_SHAPE;
  if (a->lse && (reinterpret_cast<uintptr_t>(a->lse) & 3u)) return FA_ERR_STRIDE;
  return FA_OK;
}

fa_status validate_fwd_varlen(const fa_fwd_varlen_args* a) {
  if (!a) return FA_ERR_NULL_PTR;
  if (a->B < 1 || a->Hq < 1 || a->Hkv < 1 || a->D < 1) return FA_ERR_SHAPE;
  if (a->total_q < 0 || a->total_k < 0 || a->max_seqlen_q < 0 || a->max_seqlen_q > a->total_q)
    return FA_ERR_SHAPE;
  if (a->Hq > kMaxHeads || a->Hkv > a->Hq || a->Hq % a->Hkv != 0) return FA_ERR_SHAPE;
  if (a->in_dtype != FA_BF16) return FA_ERR_DTYPE;
  if (a->out_dtype != FA_BF16 && a->out_dtype != FA_F32) return FA_ERR_DTYPE;
  if (a->D != 64 && a->D != 128) return FA_ERR_UNSUPPORTED;
  if (!scale_ok(a->scale)) return FA_ERR_ARG;
  if (a->causal != 0 && a->causal != 1) return FA_ERR_ARG;
  if (a->total_q == 0 || a->max_seqlen_q == 0) return FA_OK;
  if (!a->q || !a->o || !a->cu_seqlens_q || !a->cu_seqlens_k) return FA_ERR_NULL_PTR;
  if (a->total_k > 0 && (!a->k || !a->v)) return FA_ERR_NULL_PTR;
  const int ob = a->out_dtype == FA_BF16 ? 2 : 4;
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o))
    return FA_ERR_STRIDE;
  if (!strides_ok(a->q_stride, 2, 2) || !strides_ok(a->k_stride, 2, 2) ||
      !strides_ok(a->v_stride, 2, 2) || !strides_ok(a->o_stride, 2, ob))
    return FA_ERR_STRIDE;
  if (!pitch_ok(a->q_stride[0], 2) || !pitch_ok(a->k_stride[0], 2) || !pitch_ok(a->v_stride[0], 2))
    return FA_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(a->cu_seqlens_q) & 3u) ||
      (reinterpret_cast<uintptr_t>(a->cu_seqlens_k) & 3u))
    return FA_ERR_STRIDE;
  if (a->lse && (reinterpret_cast<uintptr_t>(a->lse) & 3u)) return FA_ERR_STRIDE;
  return FA_OK;
}

int decode_nsplit(const fa_decode_args* a) {
  return a->max_len <= 0 ? 0 : (a->max_len + a->split_len - 1) / a->split_len;
}

fa_status validate_decode(const fa_decode_args* a) {
  if (!a) return FA_ERR_NULL_PTR;
  if (a->Bs < 0 || a->Bs > kMaxGridYZ || a->Hq < 1 || a->Hkv < 1 || a->D < 1) return FA_ERR_SHAPE;
  if (a->Hq > kMaxHeads || a->Hkv > a->Hq || a->Hq % a->Hkv != 0) return FA_ERR_SHAPE;
  if (a->cache_len < 0 || a->max_len < 0 || a->max_len > a->cache_len) return FA_ERR_SHAPE;
  if (a->split_len < 128 || a->split_len % 128 != 0) return FA_ERR_SHAPE;
  if (a->in_dtype != FA_BF16) return FA_ERR_DTYPE;
  if (a->out_dtype != FA_BF16 && a->out_dtype != FA_F32) return FA_ERR_DTYPE;
  if (a->D != 64 && a->D != 128) return FA_ERR_UNSUPPORTED;
  if (!scale_ok(a->scale)) return FA_ERR_ARG;
  const int64_t nhb = (a->Hq / a->Hkv + 31) / 32;
  if ((int64_t)a->Hkv * nhb > kMaxGridYZ) return FA_ERR_SHAPE;
  if ((int64_t)decode_nsplit(a) * nhb * a->Hkv * a->Bs > 0x7fffffff) return FA_ERR_SHAPE;
  if (a->Bs == 0) return FA_OK;
  if (!a->q || !a->o || !a->seq_lens) return FA_ERR_NULL_PTR;
  if (a->max_len > 0 && (!a->k_cache || !a->v_cache)) return FA_ERR_NULL_PTR;
  const int ob = a->out_dtype == FA_BF16 ? 2 : 4;
  if (!aligned16(a->q) || !aligned16(a->o)) return FA_ERR_STRIDE;
  if (a->k_cache && !aligned16(a->k_cache)) return FA_ERR_STRIDE;
  if (a->v_cache && !aligned16(a->v_cache)) return FA_ERR_STRIDE;
  if (!strides_ok(a->q_stride, 2, 2) || !strides_ok(a->k_stride, 3, 2) ||
      !strides_ok(a->v_stride, 3, 2) || !strides_ok(a->o_stride, 2, ob))
    return FA_ERR_STRIDE;
  if (!pitch_ok(a->q_stride[1], 2) || !pitch_ok(a->k_stride[2], 2) || !pitch_ok(a->v_stride[2], 2))
    return FA_ERR_SHAPE;
  if (a->lse && (reinterpret_cast<uintptr_t>(a->lse) & 3u)) return FA_ERR_STRIDE;
  return FA_OK;
}

fa_status validate_quantize(const fa_quantize_fp8_args* a) {
  if (!a) return FA_ERR_NULL_PTR;
  if (a->B < 1 || a->H < 1 || a->N < 0 || a->D < 1) return FA_ERR_SHAPE;
  if (a->block != 64) return FA_ERR_UNSUPPORTED;
  if (a->D != 128) return FA_ERR_UNSUPPORTED;
  if (a->N == 0) return FA_OK;
  if (!a->x || !a->codes || !a->scales) return FA_ERR_NULL_PTR;
  if (!aligned16(a->x) || !aligned16(a->codes)) return FA_ERR_STRIDE;
  if (reinterpret_cast<uintptr_t>(a->scales) & 3u) return FA_ERR_STRIDE;
  if (!strides_ok(a->x_stride, 3, 2) || !strides_ok(a->codes_stride, 3, 1)) return FA_ERR_STRIDE;
  if (!pitch_ok(a->x_stride[2], 2) || !pitch_ok(a->codes_stride[2], 1)) return FA_ERR_SHAPE;
  return FA_OK;
}

fa_status validate_fwd_fp8(const fa_fwd_fp8_args* a) {
  if (!a) return FA_ERR_NULL_PTR;
  if (a->B < 1 || a->Hq < 1 || a->Hkv < 1 || a->Nq < 0 || a->Nk < 0 || a->D < 1)
    return FA_ERR_SHAPE;
  if (a->Hq > kMaxHeads || a->Hkv > a->Hq || a->Hq % a->Hkv != 0) return FA_ERR_SHAPE;
  if (a->block != 64 || a->D != 128) return FA_ERR_UNSUPPORTED;
  if (a->out_dtype != FA_BF16 && a->out_dtype != FA_F32) return FA_ERR_DTYPE;
  if (!scale_ok(a->scale)) return FA_ERR_ARG;
  if (a->causal != 0 && a->causal != 1) return FA_ERR_ARG;
  if (a->Nq == 0) return FA_OK;
  if (!a->q || !a->o || !a->q_scales) return FA_ERR_NULL_PTR;
  if (a->Nk > 0 && (!a->k || !a->v || !a->k_scales)) return FA_ERR_NULL_PTR;
  const int ob = a->out_dtype == FA_BF16 ? 2 : 4;
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o))
    return FA_ERR_STRIDE;
  if (!strides_ok(a->q_stride, 3, 1) || !strides_ok(a->k_stride, 3, 1) ||
      !strides_ok(a->v_stride, 3, 2) || !strides_ok(a->o_stride, 3, ob))
    return FA_ERR_STRIDE;
  if (!pitch_ok(a->q_stride[2], 1) || !pitch_ok(a->k_stride[2], 1) || !pitch_ok(a->v_stride[2], 2))
    return FA_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(a->q_scales) & 3u) || (reinterpret_cast<uintptr_t>(a->k_scales) & 3u))
    return FA_ERR_STRIDE;
  if (a->lse && (reinterpret_cast<uintptr_t>(a->lse) & 3u)) return FA_ERR_STRIDE;
  return FA_OK;
}

int paged_nsplit(const fa_decode_paged_args* a) {
  return a->max_len <= 0 ? 0 : (a->max_len + a->split_len - 1) / a->split_len;
}

int log2_exact(int x) {  // log2 of a power of two, else -1
  if (x <= 0 || (x & (x - 1)) != 0) return -1;
  int n = 0;
  while ((1 << n) != x) ++n;
  return n;
}

fa_status validate_decode_paged(const fa_decode_paged_args* a) {
  if (!a) return FA_ERR_NULL_PTR;
  if (a->Bs < 0 || a->Bs > kMaxGridYZ || a->Hq < 1 || a->Hkv < 1 || a->D < 1) return FA_ERR_SHAPE;
  if (a->Hq > kMaxHeads || a->Hkv > a->Hq || a->Hq % a->Hkv != 0) return FA_ERR_SHAPE;
  const int lp = log2_exact(a->page_size);
  if (lp < 4 || lp > 20) return FA_ERR_SHAPE;
  if (a->num_pages < 0 || a->max_pages_per_seq < 0 || a->max_len < 0) return FA_ERR_SHAPE;
  if ((int64_t)a->max_len > (int64_t)a->max_pages_per_seq * a->page_size) return FA_ERR_SHAPE;
  if (a->table_stride < a->max_pages_per_seq) return FA_ERR_SHAPE;
  if (a->split_len < 128 || a->split_len % 128 != 0 || a->split_len > 4096) return FA_ERR_SHAPE;
  if (a->in_dtype != FA_BF16) return FA_ERR_DTYPE;
  if (a->out_dtype != FA_BF16 && a->out_dtype != FA_F32) return FA_ERR_DTYPE;
  if (a->D != 64 && a->D != 128) return FA_ERR_UNSUPPORTED;
  if (!scale_ok(a->scale)) return FA_ERR_ARG;
  const int64_t nhb = (a->Hq / a->Hkv + 31) / 32;
  if ((int64_t)a->Hkv * nhb > kMaxGridYZ) return FA_ERR_SHAPE;
  if ((int64_t)paged_nsplit(a) * nhb * a->Hkv * a->Bs > 0x7fffffff) return FA_ERR_SHAPE;
  if (a->Bs == 0) return FA_OK;
  if (!a->q || !a->o || !a->seq_lens) return FA_ERR_NULL_PTR;
  if (a->max_len > 0 && (!a->k_pages || !a->v_pages || !a->block_table)) return FA_ERR_NULL_PTR;
  const int ob = a->out_dtype == FA_BF16 ? 2 : 4;
  if (!aligned16(a->q) || !aligned16(a->o)) return FA_ERR_STRIDE;
  if (a->k_pages && !aligned16(a->k_pages)) return FA_ERR_STRIDE;
  if (a->v_pages && !aligned16(a->v_pages)) return FA_ERR_STRIDE;
  if (!strides_ok(a->q_stride, 2, 2) || !strides_ok(a->k_stride, 3, 2) ||
      !strides_ok(a->v_stride, 3, 2) || !strides_ok(a->o_stride, 2, ob))
    return FA_ERR_STRIDE;
  if (reinterpret_cast<uintptr_t>(a->block_table) & 3u) return FA_ERR_STRIDE;
  if (!pitch_ok(a->q_stride[1], 2) || !pitch_ok(a->k_stride[2], 2) || !pitch_ok(a->v_stride[2], 2))
    return FA_ERR_SHAPE;
  // byte offsets inside one page are 32-bit
  if ((int64_t)a->page_size * a->k_stride[2] * 2 > 0x7fffffff ||
      (int64_t)a->page_size * a->v_stride[2] * 2 > 0x7fffffff)
    return FA_ERR_SHAPE;
  if (a->lse && (reinterpret_cast<uintptr_t>(a->lse) & 3u)) return FA_ERR_STRIDE;
  return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_fwd(const fa_fwd_args* a, void* stream) {
  const fa_status st = validate_fwd(a);
  if (st != FA_OK || a->Nq == 0) return st;
  fa::FwdParams p{};
  p.q = static_cast<const uint16_t*>(a->q);
  p.k = static_cast<const uint16_t*>(a->k);
  p.v = static_cast<const uint16_t*>(a->v);
  p.o = a->o;
  p.lse = a->lse;
  p.kv_lens = a->kv_lens;
  p.qs0 = a->q_stride[0], p.qs1 = a->q_stride[1], p.qs2 = a->q_stride[2];
  p.ks0 = a->k_stride[0], p.ks1 = a->k_stride[1], p.ks2 = a->k_stride[2];
  p.vs0 = a->v_stride[0], p.vs1 = a->v_stride[1], p.vs2 = a->v_stride[2];
  p.os0 = a->o_stride[0], p.os1 = a->o_stride[1], p.os2 = a->o_stride[2];
  p.lse_sb = (int64_t)a->Hq * a->Nq, p.lse_sh = a->Nq;
  p.B = a->B, p.Hq = a->Hq, p.Hkv = a->Hkv, p.Nq = a->Nq, p.Nk = a->Nk;
  p.G = a->Hq / a->Hkv;
  p.scale = a->scale;
  p.scale_log2 = a->scale * 1.4426950408889634f;
  p.causal = a->causal;
  return map_launch_error(
      fa::launch_fwd(p, a->in_dtype, a->out_dtype, a->D, static_cast<hipStream_t>(stream)));
}

// Dropout threshold t = round(256 p) in [0, 255], or -1 when p is not in [0, 1).
int dropout_threshold(float p_drop) {
  if (!(p_drop >= 0.f && p_drop < 1.f)) return -1;
  const int t = (int)std::floor(p_drop * 256.0 + 0.5);
  return t < 0 ? 0 : (t > 255 ? 255 : t);
}

fa_status fa_fwd_dropout(const fa_fwd_args* a, float p_drop, uint64_t seed, void* stream) {
  fa_status st = validate_fwd(a);
  if (st != FA_OK) return st;
  if (a->in_dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  const int t = dropout_threshold(p_drop);
  if (t < 0) return FA_ERR_ARG;
  if (t == 0) return fa_fwd(a, stream);  // nothing is dropped
  if (a->Nq == 0) return FA_OK;
  fa::FwdParams p{};
  p.q = static_cast<const uint16_t*>(a->q);
  p.k = static_cast<const uint16_t*>(a->k);
  p.v = static_cast<const uint16_t*>(a->v);
  p.o = a->o;
  p.lse = a->lse;
  p.kv_lens = a->kv_lens;
  p.qs0 = a->q_stride[0], p.qs1 = a->q_stride[1], p.qs2 = a->q_stride[2];
  p.ks0 = a->k_stride[0], p.ks1 = a->k_stride[1], p.ks2 = a->k_stride[2];
  p.vs0 = a->v_stride[0], p.vs1 = a->v_stride[1], p.vs2 = a->v_stride[2];
  p.os0 = a->o_stride[0], p.os1 = a->o_stride[1], p.os2 = a->o_stride[2];
  p.lse_sb = (int64_t)a->Hq * a->Nq, p.lse_sh = a->Nq;
  p.B = a->B, p.Hq = a->Hq, p.Hkv = a->Hkv, p.Nq = a->Nq, p.Nk = a->Nk;
  p.G = a->Hq / a->Hkv;
  p.scale = a->scale;
  p.scale_log2 = a->scale * 1.4426950408889634f;
  p.causal = a->causal;
  p.drop_t = (uint32_t)t;
  p.drop_scale = 256.f / (float)(256 - t);
  p.seed_lo = (uint32_t)(seed & 0xffffffffu), p.seed_hi = (uint32_t)(seed >> 32);
  return map_launch_error(fa::launch_fwd_dropout(p, a->out_dtype, a->D, static_cast<hipStream_t>(stream)));
}

fa_status fa_fwd_varlen(const fa_fwd_varlen_args* a, void* stream) {
  const fa_status st = validate_fwd_varlen(a);
  if (st != FA_OK || a->total_q == 0 || a->max_seqlen_q == 0) return st;
  fa::FwdParams p{};
  p.q = static_cast<const uint16_t*>(a->q);
  p.k = static_cast<const uint16_t*>(a->k);
  p.v = static_cast<const uint16_t*>(a->v);
  p.o = a->o;
  p.lse = a->lse;
  p.cu_q = a->cu_seqlens_q;
  p.cu_k = a->cu_seqlens_k;
  p.total_q = a->total_q, p.total_k = a->total_k;
  p.qs1 = a->q_stride[1], p.qs2 = a->q_stride[0];
  p.ks1 = a->k_stride[1], p.ks2 = a->k_stride[0];
  p.vs1 = a->v_stride[1], p.vs2 = a->v_stride[0];
  p.os1 = a->o_stride[1], p.os2 = a->o_stride[0];
  p.lse_sb = 0, p.lse_sh = a->total_q;
  p.B = a->B, p.Hq = a->Hq, p.Hkv = a->Hkv, p.Nq = a->max_seqlen_q, p.Nk = 0;
  p.G = a->Hq / a->Hkv;
  p.scale = a->scale;
  p.scale_log2 = a->scale * 1.4426950408889634f;
  p.causal = a->causal;
  return map_launch_error(
      fa::launch_fwd(p, a->in_dtype, a->out_dtype, a->D, static_cast<hipStream_t>(stream)));
}

size_t fa_bwd_workspace_bytes(const fa_bwd_args* a) {
  if (validate_bwd(a) != FA_OK) return 0;
  return fa::bwd_workspace_bytes(a->B, a->Hq, a->Nq, a->D);
}

namespace {
fa_status bwd_impl(const fa_bwd_args* a, int drop_t, uint64_t seed, void* workspace, size_t ws_bytes,
                   void* stream);
}

fa_status fa_bwd(const fa_bwd_args* a, void* workspace, size_t ws_bytes, void* stream) {
  return bwd_impl(a, 0, 0, workspace, ws_bytes, stream);
}

fa_status fa_bwd_dropout(const fa_bwd_args* a, float p_drop, uint64_t seed, void* workspace,
                         size_t ws_bytes, void* stream) {
  const int t = dropout_threshold(p_drop);
  if (a && t < 0) return FA_ERR_ARG;
  return bwd_impl(a, t < 0 ? 0 : t, seed, workspace, ws_bytes, stream);
}

namespace {
fa_status bwd_impl(const fa_bwd_args* a, int drop_t, uint64_t seed, void* workspace, size_t ws_bytes,
                   void* stream) {
  const fa_status st = validate_bwd(a);
  if (st != FA_OK) return st;
  if (a->Nq == 0 && a->Nk == 0) return FA_OK;
  const size_t need = fa::bwd_workspace_bytes(a->B, a->Hq, a->Nq, a->D);
  if (need > 0 && (!workspace || ws_bytes < need || !aligned16(workspace))) return FA_ERR_WORKSPACE;
  fa::BwdParams p{};
  p.q = static_cast<const uint16_t*>(a->q);
  p.k = static_cast<const uint16_t*>(a->k);
  p.v = static_cast<const uint16_t*>(a->v);
  p.o = static_cast<const uint16_t*>(a->o);
  p.dout = static_cast<const uint16_t*>(a->dout);
  p.lse = a->lse;
  p.dq = static_cast<uint16_t*>(a->dq);
  p.dk = static_cast<uint16_t*>(a->dk);
  p.dv = static_cast<uint16_t*>(a->dv);
  p.kv_lens = a->kv_lens;
  p.qs0 = a->q_stride[0], p.qs1 = a->q_stride[1], p.qs2 = a->q_stride[2];
  p.ks0 = a->k_stride[0], p.ks1 = a->k_stride[1], p.ks2 = a->k_stride[2];
  p.vs0 = a->v_stride[0], p.vs1 = a->v_stride[1], p.vs2 = a->v_stride[2];
  p.os0 = a->o_stride[0], p.os1 = a->o_stride[1], p.os2 = a->o_stride[2];
  p.dos0 = a->do_stride[0], p.dos1 = a->do_stride[1], p.dos2 = a->do_stride[2];
  p.dqs0 = a->dq_stride[0], p.dqs1 = a->dq_stride[1], p.dqs2 = a->dq_stride[2];
  p.dks0 = a->dk_stride[0], p.dks1 = a->dk_stride[1], p.dks2 = a->dk_stride[2];
  p.dvs0 = a->dv_stride[0], p.dvs1 = a->dv_stride[1], p.dvs2 = a->dv_stride[2];
  p.B = a->B, p.Hq = a->Hq, p.Hkv = a->Hkv, p.Nq = a->Nq, p.Nk = a->Nk;
  p.G = a->Hq / a->Hkv;
  p.scale = a->scale;
  p.scale_log2 = a->scale * 1.4426950408889634f;
  p.causal = a->causal;
  p.drop_t = (uint32_t)drop_t;
  p.drop_scale = drop_t > 0 ? 256.f / (float)(256 - drop_t) : 1.f;
  p.seed_lo = (uint32_t)(seed & 0xffffffffu), p.seed_hi = (uint32_t)(seed >> 32);
  fa::bwd_bind_workspace(p, workspace, a->D);
  return map_launch_error(fa::launch_bwd(p, a->D, static_cast<hipStream_t>(stream)));
}
}  // namespace

size_t fa_decode_workspace_bytes(const fa_decode_args* a) {
  if (validate_decode(a) != FA_OK) return 0;
  return fa::decode_workspace_bytes(a->Bs, a->Hq, decode_nsplit(a), a->D);
}

namespace {

// The decode launch of fa_decode and fa_decode_noalloc: `a` is valid, Bs > 0, and
// `workspace` holds at least decode_workspace_bytes() bytes.
fa_status decode_launch(const fa_decode_args* a, void* workspace, void* stream) {
  const int nsplit = decode_nsplit(a);
  fa::DecParams p{};
  p.q = static_cast<const uint16_t*>(a->q);
  p.k = static_cast<const uint16_t*>(a->k_cache);
  p.v = static_cast<const uint16_t*>(a->v_cache);
  p.seq_lens = a->seq_lens;
  p.o = a->o;
  p.lse = a->lse;
  const size_t o_bytes = ((size_t)a->Bs * a->Hq * nsplit * a->D * 4 + 255) & ~size_t(255);
  p.part_o = static_cast<float*>(workspace);
  p.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + o_bytes);
  p.qs0 = a->q_stride[0], p.qs1 = a->q_stride[1];
  p.ks0 = a->k_stride[0], p.ks1 = a->k_stride[1], p.ks2 = a->k_stride[2];
  p.vs0 = a->v_stride[0], p.vs1 = a->v_stride[1], p.vs2 = a->v_stride[2];
  p.os0 = a->o_stride[0], p.os1 = a->o_stride[1];
  p.Bs = a->Bs, p.Hq = a->Hq, p.Hkv = a->Hkv;
  p.G = a->Hq / a->Hkv;
  p.nhb = (p.G + 31) / 32;
  p.max_len = a->max_len, p.split_len = a->split_len, p.nsplit = nsplit;
  p.scale = a->scale;
  p.scale_log2 = a->scale * 1.4426950408889634f;
  return map_launch_error(
      fa::launch_decode(p, a->D, a->out_dtype, static_cast<hipStream_t>(stream)));
}

}  // namespace

fa_status fa_decode(const fa_decode_args* a, void* workspace, size_t ws_bytes, void* stream) {
  const fa_status st = validate_decode(a);
  if (st != FA_OK || a->Bs == 0) return st;
  const size_t need = fa::decode_workspace_bytes(a->Bs, a->Hq, decode_nsplit(a), a->D);
  if (need > 0 && (!workspace || ws_bytes < need || !aligned16(workspace))) return FA_ERR_WORKSPACE;
  return decode_launch(a, workspace, stream);
}

fa_status fa_decode_noalloc(const fa_decode_args* a, void* stream) {
  const fa_status st = validate_decode(a);
  if (st != FA_OK || a->Bs == 0) return st;
  const size_t need = fa::decode_workspace_bytes(a->Bs, a->Hq, decode_nsplit(a), a->D);
  if (need > fa::kDecodeScratchBytes) return FA_ERR_WORKSPACE;
  void* scratch = nullptr;
  const hipError_t e = fa::decode_scratch(&scratch);
  if (e != hipSuccess) return FA_ERR_DEVICE;  // no current device, or its array has no address
  return decode_launch(a, scratch, stream);
}

fa_status fa_quantize_fp8(const fa_quantize_fp8_args* a, void* stream) {
  const fa_status st = validate_quantize(a);
  if (st != FA_OK || a->N == 0) return st;
  fa::QuantParams p{};
  p.x = static_cast<const uint16_t*>(a->x);
  p.codes = static_cast<uint8_t*>(a->codes);
  p.scales = a->scales;
  p.xs0 = a->x_stride[0], p.xs1 = a->x_stride[1], p.xs2 = a->x_stride[2];
  p.cs0 = a->codes_stride[0], p.cs1 = a->codes_stride[1], p.cs2 = a->codes_stride[2];
  p.B = a->B, p.H = a->H, p.N = a->N;
  p.nb = (a->N + a->block - 1) / a->block;
  return map_launch_error(fa::launch_quantize_fp8(p, a->D, static_cast<hipStream_t>(stream)));
}

fa_status fa_fwd_fp8(const fa_fwd_fp8_args* a, void* stream) {
  const fa_status st = validate_fwd_fp8(a);
  if (st != FA_OK || a->Nq == 0) return st;
  fa::FwdParams p{};
  p.q = static_cast<const uint16_t*>(a->q);  // E4M3 codes; strides below are in bytes
  p.k = static_cast<const uint16_t*>(a->k);
  p.v = static_cast<const uint16_t*>(a->v);
  p.o = a->o;
  p.lse = a->lse;
  p.kv_lens = a->kv_lens;
  p.q_scale = a->q_scales;
  p.k_scale = a->k_scales;
  const int nqb = (a->Nq + 63) / 64, nkb = (a->Nk + 63) / 64;
  p.qsc_b = (int64_t)a->Hq * nqb, p.qsc_h = nqb;
  p.ksc_b = (int64_t)a->Hkv * nkb, p.ksc_h = nkb;
  p.qs0 = a->q_stride[0], p.qs1 = a->q_stride[1], p.qs2 = a->q_stride[2];
  p.ks0 = a->k_stride[0], p.ks1 = a->k_stride[1], p.ks2 = a->k_stride[2];
  p.vs0 = a->v_stride[0], p.vs1 = a->v_stride[1], p.vs2 = a->v_stride[2];
  p.os0 = a->o_stride[0], p.os1 = a->o_stride[1], p.os2 = a->o_stride[2];
  p.lse_sb = (int64_t)a->Hq * a->Nq, p.lse_sh = a->Nq;
  p.B = a->B, p.Hq = a->Hq, p.Hkv = a->Hkv, p.Nq = a->Nq, p.Nk = a->Nk;
  p.G = a->Hq / a->Hkv;
  p.scale = a->scale;
  p.scale_log2 = a->scale * 1.4426950408889634f;
  p.causal = a->causal;
  return map_launch_error(fa::launch_fwd_fp8(p, a->out_dtype, static_cast<hipStream_t>(stream)));
}

size_t fa_decode_paged_workspace_bytes(const fa_decode_paged_args* a) {
  if (validate_decode_paged(a) != FA_OK) return 0;
  return fa::decode_workspace_bytes(a->Bs, a->Hq, paged_nsplit(a), a->D);
}

fa_status fa_decode_paged(const fa_decode_paged_args* a, void* workspace, size_t ws_bytes,
                          void* stream) {
  const fa_status st = validate_decode_paged(a);
  if (st != FA_OK || a->Bs == 0) return st;
  const int nsplit = paged_nsplit(a);
  const size_t need = fa::decode_workspace_bytes(a->Bs, a->Hq, nsplit, a->D);
  if (need > 0 && (!workspace || ws_bytes < need || !aligned16(workspace))) return FA_ERR_WORKSPACE;
  fa::DecParams p{};
  p.q = static_cast<const uint16_t*>(a->q);
  p.k = static_cast<const uint16_t*>(a->k_pages);
  p.v = static_cast<const uint16_t*>(a->v_pages);
  p.seq_lens = a->seq_lens;
  p.o = a->o;
  p.lse = a->lse;
  const size_t o_bytes = ((size_t)a->Bs * a->Hq * nsplit * a->D * 4 + 255) & ~size_t(255);
  p.part_o = static_cast<float*>(workspace);
  p.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + o_bytes);
  p.qs0 = a->q_stride[0], p.qs1 = a->q_stride[1];
  p.ks0 = a->k_stride[0], p.ks1 = a->k_stride[1], p.ks2 = a->k_stride[2];
  p.vs0 = a->v_stride[0], p.vs1 = a->v_stride[1], p.vs2 = a->v_stride[2];
  p.os0 = a->o_stride[0], p.os1 = a->o_stride[1];
  p.Bs = a->Bs, p.Hq = a->Hq, p.Hkv = a->Hkv;
  p.G = a->Hq / a->Hkv;
  p.nhb = (p.G + 31) / 32;
  p.max_len = a->max_len, p.split_len = a->split_len, p.nsplit = nsplit;
  p.scale = a->scale;
  p.scale_log2 = a->scale * 1.4426950408889634f;
  p.table = a->block_table;
  p.table_stride = a->table_stride;
  p.page_shift = log2_exact(a->page_size);
  p.num_pages = a->num_pages;
  return map_launch_error(
      fa::launch_decode(p, a->D, a->out_dtype, static_cast<hipStream_t>(stream)));
}

const char* fa_status_str(int s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL_PTR: return "FA_ERR_NULL_PTR: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: a size is out of range or inconsistent";
    case FA_ERR_DTYPE: return "FA_ERR_DTYPE: unsupported dtype combination";
    case FA_ERR_STRIDE: return "FA_ERR_STRIDE: stride or pointer not 16-byte aligned";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head dim or mode not built";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
    case FA_ERR_DEVICE: return "FA_ERR_DEVICE: no usable gfx950 device";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH: kernel launch failed";
    case FA_ERR_ARG: return "FA_ERR_ARG: invalid scalar argument";
    default: return "FA_ERR_UNKNOWN";
  }
}

int fa_device_supported(int device) {
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return 0;
  return std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
}

int fa_version(void) { return (1 << 16) | 1; }

}  // extern "C"
