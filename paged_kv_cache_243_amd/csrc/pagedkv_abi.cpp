// pagedkv_abi.cpp -- the C ABI of libpagedkv.so: argument validation, workspace
// sizing and dispatch onto the gfx950 kernels.  Declarations and the contract of
// every entry point are in include/pagedkv.h.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "kernels.h"
#include "pagedkv.h"
#include "pagedkv_host.h"

using pkv::AttnParams;
using pkv::WriteParams;

namespace {

constexpr int kPageSize = 16;
constexpr int kMaxGroup = 16;
constexpr int kMaxSplitTokens = 4096;

int64_t numel(const pkv_tensor* t) {
  int64_t n = 1;
  for (int i = 0; i < t->ndim; ++i) n *= t->shape[i];
  return n;
}

int elem_bytes(int32_t dtype) {
  switch (dtype) {
    case PKV_F32: return 4;
    case PKV_BF16: return 2;
    case PKV_FP8_E4M3FN: return 1;
    case PKV_I64: return 8;
    default: return 0;
  }
}

// rank, non-negative sizes, non-NULL data when non-empty, alignment
int check_tensor(const pkv_tensor* t, int ndim, size_t align) {
  if (t == nullptr) return PKV_ERR_NULL;
  if (t->ndim != ndim) return PKV_ERR_SHAPE;
  for (int i = 0; i < ndim; ++i)
    if (t->shape[i] < 0) return PKV_ERR_SHAPE;
  if (elem_bytes(t->dtype) == 0) return PKV_ERR_DTYPE;
  if (numel(t) > 0) {
    if (t->data == nullptr) return PKV_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(t->data) % align != 0) return PKV_ERR_UNSUPPORTED;
  }
  return PKV_OK;
}

bool same_shape(const pkv_tensor* a, const pkv_tensor* b) {
  if (a->ndim != b->ndim) return false;
  for (int i = 0; i < a->ndim; ++i)
    if (a->shape[i] != b->shape[i]) return false;
  return true;
}

#define PKV_TRY(expr)            \
  do {                           \
    int _st = (expr);            \
    if (_st != PKV_OK) return _st; \
  } while (0)

constexpr int kMaxDevices = 64;

// The device `stream` runs on (the current device for the null stream), or -1.
int stream_device(hipStream_t stream) {
  int dev = -1;
  if (stream != nullptr) {
    hipDevice_t d;
    if (hipStreamGetDevice(stream, &d) == hipSuccess) dev = (int)d;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    dev = -1;
  }
  return dev >= 0 && dev < kMaxDevices ? dev : -1;
}

// Compute units of device `dev` (cached per device); 256, MI355X's count, when
// the device cannot be queried.
int device_cu_count(int dev) {
  static int cached[kMaxDevices] = {0};
  if (dev < 0 || dev >= kMaxDevices) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

struct AttnPlan {
  AttnParams p;
  enum { kNone, kF32, kDecode, kPrefill } kernel;
  size_t workspace;
  int slot_parts;  // decode: partition ranges the partial slots are sized for
};

// Validates the attention arguments and fills the launch plan (no HIP calls).
// n_cu > 0 fixes the decode grid for a device of that many CUs (0: a size
// query, no grid); `tight` sizes the decode partials for that grid instead of
// for any device.
int plan_attention(const pkv_tensor* q, const pkv_tensor* key_pool, const pkv_tensor* value_pool,
                   const pkv_tensor* block_table, const pkv_tensor* seq_lens,
                   const pkv_tensor* query_start_loc, float scale, const pkv_tensor* out,
                   const pkv_attn_opts* opts, bool check_runtime_args, int n_cu, bool tight,
                   AttnPlan& plan) {
  PKV_TRY(check_tensor(q, 3, 16));
  PKV_TRY(check_tensor(key_pool, 4, 16));
  if (value_pool) PKV_TRY(check_tensor(value_pool, 4, 16));
  PKV_TRY(check_tensor(block_table, 2, 8));
  if (check_runtime_args) {
    PKV_TRY(check_tensor(seq_lens, 1, 8));
    PKV_TRY(check_tensor(query_start_loc, 1, 8));
    PKV_TRY(check_tensor(out, 3, 16));
    if (value_pool == nullptr) return PKV_ERR_NULL;
  }
  const int64_t T = q->shape[0], Hq = q->shape[1], D = q->shape[2];
  const int64_t num_pages = key_pool->shape[0], ps = key_pool->shape[1];
  const int64_t Hkv = key_pool->shape[2];
  const int64_t B = block_table->shape[0], max_blocks = block_table->shape[1];

  // element types
  if (q->dtype != PKV_F32 && q->dtype != PKV_BF16) return PKV_ERR_DTYPE;
  const int kv = key_pool->dtype;
  if (kv != PKV_F32 && kv != PKV_BF16 && kv != PKV_FP8_E4M3FN) return PKV_ERR_DTYPE;
  if (value_pool && value_pool->dtype != kv) return PKV_ERR_DTYPE;
  if ((q->dtype == PKV_F32) != (kv == PKV_F32)) return PKV_ERR_DTYPE;
  if (block_table->dtype != PKV_I64) return PKV_ERR_DTYPE;
  if (check_runtime_args) {
    if (seq_lens->dtype != PKV_I64 || query_start_loc->dtype != PKV_I64) return PKV_ERR_DTYPE;
    if (out->dtype != q->dtype) return PKV_ERR_DTYPE;
  }

  // shapes
  if (key_pool->shape[3] != D) return PKV_ERR_SHAPE;
  if (value_pool && !same_shape(key_pool, value_pool)) return PKV_ERR_SHAPE;
  if (check_runtime_args) {
    if (!same_shape(q, out)) return PKV_ERR_SHAPE;
    if (seq_lens->shape[0] != B) return PKV_ERR_SHAPE;
    if (query_start_loc->shape[0] != B + 1) return PKV_ERR_SHAPE;
  }
  if (Hkv <= 0 || Hq <= 0) return PKV_ERR_SHAPE;
  if (Hq % Hkv != 0) return PKV_ERR_SHAPE;

  // supported geometry
  const int64_t G = Hq / Hkv;
  if (ps != kPageSize) return PKV_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return PKV_ERR_UNSUPPORTED;
  if (G > kMaxGroup) return PKV_ERR_UNSUPPORTED;
  if (num_pages > INT32_MAX) return PKV_ERR_UNSUPPORTED;
  if (B > 65535 || Hkv > 65535) return PKV_ERR_UNSUPPORTED;

  // options
  if (check_runtime_args && !std::isfinite(scale)) return PKV_ERR_SCALE;
  const bool fp8 = kv == PKV_FP8_E4M3FN;
  if (check_runtime_args) {
    const bool has_scales = opts && opts->k_scale && opts->v_scale;
    const bool any_scale = opts && (opts->k_scale || opts->v_scale);
    if (fp8 && !has_scales) return PKV_ERR_SCALE;
    if (!fp8 && any_scale) return PKV_ERR_SCALE;
  }
  int64_t max_q = opts ? opts->max_query_len : 0;
  if (max_q < 0) return PKV_ERR_SHAPE;
  if (max_q == 0 || max_q > T) max_q = T;
  int split = opts ? opts->split_tokens : 0;
  if (split < 0 || split % kPageSize != 0 || split > kMaxSplitTokens) return PKV_ERR_UNSUPPORTED;
  const int64_t shared_pages = opts ? opts->shared_prefix_pages : 0;
  if (shared_pages < 0) return PKV_ERR_SHAPE;
  if (shared_pages % 2 != 0 || shared_pages > max_blocks) return PKV_ERR_UNSUPPORTED;

  AttnParams& p = plan.p;
  memset(&p, 0, sizeof p);
  p.q = q->data;
  p.out = out ? out->data : nullptr;
  p.key_pool = key_pool->data;
  p.value_pool = value_pool ? value_pool->data : nullptr;
  p.block_table = (const int64_t*)block_table->data;
  p.seq_lens = seq_lens ? (const int64_t*)seq_lens->data : nullptr;
  p.qsl = query_start_loc ? (const int64_t*)query_start_loc->data : nullptr;
  p.k_scale = opts ? opts->k_scale : nullptr;
  p.v_scale = opts ? opts->v_scale : nullptr;
  p.T = T;
  p.B = B;
  p.max_blocks = max_blocks;
  p.num_pages = num_pages;
  p.Hq = (int)Hq;
  p.Hkv = (int)Hkv;
  p.D = (int)D;
  p.G = (int)G;
  p.scale = scale;
  p.kv_type = kv == PKV_F32 ? pkv::KV_F32 : (fp8 ? pkv::KV_FP8 : pkv::KV_BF16);
  p.kv_bytes = elem_bytes(kv);
  p.max_query_len = (int)std::min<int64_t>(max_q, INT32_MAX);

  plan.workspace = 0;
  if (T == 0 || B == 0) {
    plan.kernel = AttnPlan::kNone;
  } else if (kv == PKV_F32) {
    plan.kernel = AttnPlan::kF32;
    if (shared_pages > 0) return PKV_ERR_UNSUPPORTED;
  } else if (max_q == 1) {
    plan.kernel = AttnPlan::kDecode;
    if (B > pkv::kDecodeMaxSeqs) return PKV_ERR_UNSUPPORTED;
    // the decode kernel counts 32-position units of all sequences in 32 bits
    if (B * ((max_blocks * kPageSize + 31) / 32) > INT32_MAX) return PKV_ERR_UNSUPPORTED;
    p.split_tokens = split;
    // with a shared prefix, the decode grid takes the CUs its items leave
    size_t prefix_bytes = 0;
    int decode_cu = n_cu;
    if (shared_pages > 0) {
      prefix_bytes = pkv::prefix_plan(p, shared_pages * kPageSize, n_cu, tight);
      if (n_cu > 0) decode_cu = std::max(n_cu - p.prefix_wgs, n_cu / 4);
    }
    if (n_cu > 0) p.grid_parts = pkv::decode_grid_parts(B, max_blocks * kPageSize, split, decode_cu, (int)Hkv);
    p.decode_rounds = pkv::decode_rounds(p.grid_parts, decode_cu, (int)Hkv);
    plan.slot_parts = tight ? p.grid_parts : pkv::kDecodeMaxParts;
    plan.workspace = pkv::decode_workspace_bytes(B, (int)Hq, (int)D, plan.slot_parts) + prefix_bytes;
  } else {
    plan.kernel = AttnPlan::kPrefill;
    if (shared_pages > 0) return PKV_ERR_UNSUPPORTED;
    // the prefill kernels index positions with 32-bit integers and its work
    // list packs (sequence, query tile) into 16 + 16 bits
    const int64_t tpt = pkv::prefill_tokens_per_tile((int)G);
    if (max_blocks * kPageSize > INT32_MAX) return PKV_ERR_UNSUPPORTED;
    if ((T + tpt - 1) / tpt > 65535) return PKV_ERR_UNSUPPORTED;
    pkv::prefill_split_plan(p);
    // a workgroup of 512 threads per (query tile, key chunk, KV head): the
    // launch's work-items must stay below 2^32
    if (p.plan_tiles_cap * p.split_max_chunks * Hkv > pkv::kPrefillMaxGroups) return PKV_ERR_UNSUPPORTED;
    plan.workspace = pkv::prefill_workspace_bytes(p);
  }
  return PKV_OK;
}

// Enqueues the planned attention with its workspace at `ws`.
int launch_attention(AttnPlan& plan, void* ws, const pkv_attn_opts* opts, hipStream_t s) {
  AttnParams& p = plan.p;
  hipError_t err = hipSuccess;
  pkv::LaunchEvents ev;
  if (opts) {
    ev.begin = (hipEvent_t)opts->timing_events[0];
    ev.end = (hipEvent_t)opts->timing_events[1];
  }
  switch (plan.kernel) {
    case AttnPlan::kNone:
      return PKV_OK;
    case AttnPlan::kF32:
      err = pkv::launch_attention_f32(p, s, ev);
      break;
    case AttnPlan::kDecode:
      pkv::decode_workspace_carve(p, ws, plan.slot_parts);
      if (p.prefix_len > 0)
        pkv::prefix_workspace_carve(p, (char*)ws + pkv::decode_workspace_bytes(p.B, p.Hq, p.D, plan.slot_parts));
      err = pkv::launch_decode(p, s, ev);
      break;
    case AttnPlan::kPrefill:
      pkv::prefill_workspace_carve(p, ws);
      err = pkv::launch_prefill(p, s, ev);
      break;
  }
  return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

}  // namespace

namespace pkv {

// paged_attention with its workspace in a fixed region of `region_bytes`
// bytes that `region(device)` resolves for the stream's device; the region is
// resolved only once the arguments are known to fit in it.  The decode
// partials are sized for this device's own grid.
int attention_in_region(const pkv_tensor* q, const pkv_tensor* key_pool, const pkv_tensor* value_pool,
                        const pkv_tensor* block_table, const pkv_tensor* seq_lens,
                        const pkv_tensor* query_start_loc, float scale, pkv_tensor* out,
                        const pkv_attn_opts* opts, size_t region_bytes, void* (*region)(int device),
                        void* stream) {
  if (opts && (opts->workspace || opts->workspace_bytes)) return PKV_ERR_WORKSPACE;
  const hipStream_t s = (hipStream_t)stream;
  const int dev = stream_device(s);
  AttnPlan plan;
  PKV_TRY(plan_attention(q, key_pool, value_pool, block_table, seq_lens, query_start_loc, scale, out, opts,
                         true, device_cu_count(dev), true, plan));
  if (plan.workspace > region_bytes) return PKV_ERR_SCRATCH;
  void* ws = nullptr;
  if (plan.workspace > 0) {
    if (dev < 0) return PKV_ERR_HIP;
    ws = region(dev);
    if (ws == nullptr) return PKV_ERR_HIP;
  }
  return launch_attention(plan, ws, opts, s);
}

}  // namespace pkv

extern "C" {

int pkv_abi_version(void) { return 4; }

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "required pointer is NULL";
    case PKV_ERR_SHAPE: return "shape mismatch";
    case PKV_ERR_DTYPE: return "element type not allowed";
    case PKV_ERR_UNSUPPORTED: return "unsupported geometry or alignment";
    case PKV_ERR_SCALE: return "bad scale (non-finite, or fp8 pool without k/v scales)";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_HIP: return "HIP runtime error";
    case PKV_ERR_INDEX: return "index value out of range";
    case PKV_ERR_SCRATCH:
      return "the call needs more workspace than the fixed scratch of paged_attention_noalloc "
             "(PKV_NOALLOC_SCRATCH_BYTES); use paged_attention with a caller workspace";
    case PKV_ERR_NO_PAGES: return "too few free pages";
    case PKV_ERR_BAD_HANDLE: return "stale or unknown handle, or a page released more often than held";
    case PKV_ERR_DIRTY: return "a page to describe is dirty (not confirmed overwritten since it was freed)";
    default: return "unknown status";
  }
}

}  // extern "C"

namespace {

// Argument checks of the write; fills its launch parameters.
int plan_write(const pkv_tensor* k, const pkv_tensor* v, const pkv_tensor* slot_mapping,
               const pkv_tensor* key_pool, const pkv_tensor* value_pool, WriteParams& p) {
  PKV_TRY(check_tensor(k, 3, 16));
  PKV_TRY(check_tensor(v, 3, 16));
  PKV_TRY(check_tensor(slot_mapping, 1, 8));
  PKV_TRY(check_tensor(key_pool, 4, 16));
  PKV_TRY(check_tensor(value_pool, 4, 16));
  const int kv = key_pool->dtype;
  if (kv != PKV_F32 && kv != PKV_BF16 && kv != PKV_FP8_E4M3FN) return PKV_ERR_DTYPE;
  if (value_pool->dtype != kv || k->dtype != kv || v->dtype != kv) return PKV_ERR_DTYPE;
  if (slot_mapping->dtype != PKV_I64) return PKV_ERR_DTYPE;
  if (!same_shape(key_pool, value_pool) || !same_shape(k, v)) return PKV_ERR_SHAPE;
  if (slot_mapping->shape[0] != k->shape[0]) return PKV_ERR_SHAPE;
  if (k->shape[1] != key_pool->shape[2] || k->shape[2] != key_pool->shape[3]) return PKV_ERR_SHAPE;
  const int64_t row_bytes = key_pool->shape[2] * key_pool->shape[3] * elem_bytes(kv);
  if (row_bytes <= 0 || row_bytes % 16 != 0) return PKV_ERR_UNSUPPORTED;
  p.k = k->data;
  p.v = v->data;
  p.slots = (const int64_t*)slot_mapping->data;
  p.key_pool = key_pool->data;
  p.value_pool = value_pool->data;
  p.n_tokens = k->shape[0];
  p.row_bytes = row_bytes;
  return PKV_OK;
}

}  // namespace

extern "C" {

int paged_kv_write(const pkv_tensor* k, const pkv_tensor* v, const pkv_tensor* slot_mapping,
                   pkv_tensor* key_pool, pkv_tensor* value_pool, void* stream) {
  WriteParams p;
  PKV_TRY(plan_write(k, v, slot_mapping, key_pool, value_pool, p));
  if (p.n_tokens == 0) return PKV_OK;
  return pkv::launch_write(p, (hipStream_t)stream) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int paged_kv_write_fp8(const pkv_tensor* k, const pkv_tensor* v, const pkv_tensor* slot_mapping,
                       pkv_tensor* key_pool, pkv_tensor* value_pool, const float* k_scale,
                       const float* v_scale, void* stream) {
  PKV_TRY(check_tensor(k, 3, 16));
  PKV_TRY(check_tensor(v, 3, 16));
  PKV_TRY(check_tensor(slot_mapping, 1, 8));
  PKV_TRY(check_tensor(key_pool, 4, 8));
  PKV_TRY(check_tensor(value_pool, 4, 8));
  if (k->dtype != PKV_BF16 || v->dtype != PKV_BF16) return PKV_ERR_DTYPE;
  if (key_pool->dtype != PKV_FP8_E4M3FN || value_pool->dtype != PKV_FP8_E4M3FN) return PKV_ERR_DTYPE;
  if (slot_mapping->dtype != PKV_I64) return PKV_ERR_DTYPE;
  if (!same_shape(key_pool, value_pool) || !same_shape(k, v)) return PKV_ERR_SHAPE;
  if (slot_mapping->shape[0] != k->shape[0]) return PKV_ERR_SHAPE;
  if (k->shape[1] != key_pool->shape[2] || k->shape[2] != key_pool->shape[3]) return PKV_ERR_SHAPE;
  if (!k_scale || !v_scale) return PKV_ERR_SCALE;
  if (key_pool->shape[3] <= 0 || key_pool->shape[3] % 8 != 0 || key_pool->shape[2] <= 0) return PKV_ERR_UNSUPPORTED;
  pkv::WriteFp8Params p;
  p.k = k->data;
  p.v = v->data;
  p.slots = (const int64_t*)slot_mapping->data;
  p.key_pool = key_pool->data;
  p.value_pool = value_pool->data;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.n_tokens = k->shape[0];
  p.Hkv = key_pool->shape[2];
  p.D = key_pool->shape[3];
  if (p.n_tokens == 0) return PKV_OK;
  return pkv::launch_write_fp8(p, (hipStream_t)stream) == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int paged_block_table_from_csr(const pkv_tensor* kv_indptr, const pkv_tensor* kv_indices,
                               const pkv_tensor* kv_last_page_len, int64_t page_size, int64_t pad_page,
                               pkv_tensor* block_table, pkv_tensor* seq_lens, void* stream) {
  PKV_TRY(check_tensor(kv_indptr, 1, 8));
  PKV_TRY(check_tensor(kv_indices, 1, 8));
  PKV_TRY(check_tensor(kv_last_page_len, 1, 8));
  PKV_TRY(check_tensor(block_table, 2, 8));
  PKV_TRY(check_tensor(seq_lens, 1, 8));
  if (kv_indptr->dtype != PKV_I64 || kv_indices->dtype != PKV_I64 || kv_last_page_len->dtype != PKV_I64 ||
      block_table->dtype != PKV_I64 || seq_lens->dtype != PKV_I64)
    return PKV_ERR_DTYPE;
  const int64_t B = block_table->shape[0], max_blocks = block_table->shape[1];
  if (kv_indptr->shape[0] != B + 1 || kv_last_page_len->shape[0] != B || seq_lens->shape[0] != B)
    return PKV_ERR_SHAPE;
  if (page_size <= 0) return PKV_ERR_SHAPE;
  if (B == 0 || max_blocks == 0) {
    if (B > 0 && max_blocks == 0) return PKV_ERR_SHAPE;  // lengths need a row to live in
    return PKV_OK;
  }
  return pkv::launch_csr_to_block_table((const int64_t*)kv_indptr->data, (const int64_t*)kv_indices->data,
                                        (const int64_t*)kv_last_page_len->data, kv_indices->shape[0], B, max_blocks,
                                        page_size, pad_page,
                                        (int64_t*)block_table->data, (int64_t*)seq_lens->data,
                                        (hipStream_t)stream) == hipSuccess
             ? PKV_OK
             : PKV_ERR_HIP;
}

size_t paged_attention_workspace_size(const pkv_tensor* q, const pkv_tensor* key_pool,
                                      const pkv_tensor* block_table, const pkv_attn_opts* opts) {
  AttnPlan plan;
  if (plan_attention(q, key_pool, nullptr, block_table, nullptr, nullptr, 1.0f, nullptr, opts,
                     false, 0, false, plan) != PKV_OK)
    return (size_t)-1;
  return plan.workspace;
}

int paged_attention(const pkv_tensor* q, const pkv_tensor* key_pool, const pkv_tensor* value_pool,
                    const pkv_tensor* block_table, const pkv_tensor* seq_lens,
                    const pkv_tensor* query_start_loc, float scale, pkv_tensor* out,
                    const pkv_attn_opts* opts, void* stream) {
  const hipStream_t s = (hipStream_t)stream;
  AttnPlan plan;
  PKV_TRY(plan_attention(q, key_pool, value_pool, block_table, seq_lens, query_start_loc, scale,
                         out, opts, true, device_cu_count(stream_device(s)), false, plan));
  if (plan.workspace > 0) {
    if (!opts || !opts->workspace) return PKV_ERR_WORKSPACE;
    if (opts->workspace_bytes < plan.workspace) return PKV_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(opts->workspace) % 16 != 0) return PKV_ERR_WORKSPACE;
  }
  return launch_attention(plan, opts ? opts->workspace : nullptr, opts, s);
}

int paged_kv_write_attention(const pkv_tensor* k, const pkv_tensor* v, const pkv_tensor* slot_mapping,
                             pkv_tensor* key_pool, pkv_tensor* value_pool, const pkv_tensor* q,
                             const pkv_tensor* block_table, const pkv_tensor* seq_lens,
                             const pkv_tensor* query_start_loc, float scale, pkv_tensor* out,
                             const pkv_attn_opts* opts, void* stream) {
  const hipStream_t s = (hipStream_t)stream;
  WriteParams wp;
  PKV_TRY(plan_write(k, v, slot_mapping, key_pool, value_pool, wp));
  AttnPlan plan;
  PKV_TRY(plan_attention(q, key_pool, value_pool, block_table, seq_lens, query_start_loc, scale, out, opts, true,
                         device_cu_count(stream_device(s)), false, plan));
  if (plan.workspace > 0) {
    if (!opts || !opts->workspace) return PKV_ERR_WORKSPACE;
    if (opts->workspace_bytes < plan.workspace) return PKV_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(opts->workspace) % 16 != 0) return PKV_ERR_WORKSPACE;
  }
  void* ws = opts ? opts->workspace : nullptr;
  if (plan.kernel == AttnPlan::kDecode && wp.n_tokens == q->shape[0] &&
      pkv::decode_can_fuse_write(plan.p, wp.n_tokens, wp.row_bytes)) {
    // a decode step whose new rows are the query rows' keys: one kernel
    // writes them and attends, taking each sequence's last key from them
    plan.p.new_k = wp.k;
    plan.p.new_v = wp.v;
    plan.p.new_slots = wp.slots;
    plan.p.n_new = wp.n_tokens;
    return launch_attention(plan, ws, opts, s);
  }
  if (wp.n_tokens > 0 && pkv::launch_write(wp, s) != hipSuccess) return PKV_ERR_HIP;
  return launch_attention(plan, ws, opts, s);
}

// Host-memory form of the metadata check; paged_validate_metadata copies the
// device tensors and calls it.
int pkv_check_metadata_host(const int64_t* slots, int64_t n_slots, const int64_t* block_table,
                            int64_t B, int64_t max_blocks, const int64_t* seq_lens,
                            const int64_t* qsl, int64_t num_pages, int64_t page_size,
                            int64_t num_query_rows, int64_t shared_prefix_pages, uint32_t checks,
                            char* message, size_t message_len) {
  auto fail = [&](const char* fmt, long long a, long long b) {
    if (message && message_len) snprintf(message, message_len, fmt, a, b);
    return PKV_ERR_INDEX;
  };
  if (page_size <= 0 || num_pages < 0 || shared_prefix_pages < 0) return PKV_ERR_SHAPE;
  const int64_t capacity = num_pages * page_size;
  if (slots) {
    std::vector<int64_t> seen;
    seen.reserve((size_t)n_slots);
    for (int64_t t = 0; t < n_slots; ++t) {
      if (slots[t] < -1 || slots[t] >= capacity)
        return fail("slot_mapping[%lld] = %lld is out of range", (long long)t, (long long)slots[t]);
      if (slots[t] >= 0) seen.push_back(slots[t]);
    }
    std::sort(seen.begin(), seen.end());
    for (size_t i = 1; i < seen.size(); ++i)
      if (seen[i] == seen[i - 1]) return fail("slot %lld appears twice (%lld)", (long long)seen[i], 2);
  }
  if (qsl[0] != 0) return fail("query_start_loc[%lld] = %lld, expected 0", 0, (long long)qsl[0]);
  if (qsl[B] != num_query_rows)
    return fail("query_start_loc[B] = %lld, expected T = %lld", (long long)qsl[B], (long long)num_query_rows);
  for (int64_t b = 0; b < B; ++b) {
    const int64_t n = qsl[b + 1] - qsl[b];
    if (n < 0) return fail("query_start_loc decreases at %lld (%lld)", (long long)b, (long long)n);
    if (n > seq_lens[b]) return fail("sequence %lld has more query rows than keys (%lld)", (long long)b, (long long)n);
    if (seq_lens[b] > max_blocks * page_size)
      return fail("seq_lens[%lld] = %lld exceeds the block table", (long long)b, (long long)seq_lens[b]);
    const int64_t nblk = (seq_lens[b] + page_size - 1) / page_size;
    for (int64_t j = 0; j < nblk; ++j) {
      const int64_t pg = block_table[b * max_blocks + j];
      if (pg < 0 || pg >= num_pages)
        return fail("block_table[%lld] names page %lld, out of range", (long long)(b * max_blocks + j), (long long)pg);
    }
  }
  // a shared-prefix statement: every sequence with a query row holds more
  // positions than the prefix, and its row starts with the same pages as the
  // first such sequence's row
  if (shared_prefix_pages > 0) {
    if (shared_prefix_pages > max_blocks)
      return fail("shared_prefix_pages = %lld exceeds the block table width %lld", (long long)shared_prefix_pages,
                  (long long)max_blocks);
    int64_t b0 = -1;
    for (int64_t b = 0; b < B; ++b) {
      if (qsl[b + 1] == qsl[b]) continue;
      if (seq_lens[b] <= shared_prefix_pages * page_size)
        return fail("sequence %lld holds %lld positions, not more than the shared prefix", (long long)b,
                    (long long)seq_lens[b]);
      if (b0 < 0) {
        b0 = b;
        continue;
      }
      for (int64_t j = 0; j < shared_prefix_pages; ++j)
        if (block_table[b * max_blocks + j] != block_table[b0 * max_blocks + j])
          return fail("sequence %lld does not share prefix page %lld", (long long)b, (long long)j);
    }
  }
  // the fused write + attention's statement: new row t is the key of query
  // row t, stored at the slot of that row's position, and no sequence reads a
  // slot this step writes at any other position
  if (checks & PKV_CHECK_NEW_ROWS_ARE_QUERY_ROWS) {
    if (!slots) return fail("the new-rows check needs slot_mapping (%lld, %lld)", 0, 0);
    if (n_slots != num_query_rows)
      return fail("slot_mapping has %lld rows, not the %lld query rows", (long long)n_slots, (long long)num_query_rows);
    auto slot_of = [&](int64_t b, int64_t pos) {
      return block_table[b * max_blocks + pos / page_size] * page_size + pos % page_size;
    };
    for (int64_t b = 0; b < B; ++b) {
      const int64_t n = qsl[b + 1] - qsl[b], L = seq_lens[b];
      for (int64_t i = 0; i < n; ++i)
        if (slots[qsl[b] + i] != slot_of(b, L - n + i))
          return fail("slot_mapping[%lld] = %lld is not the slot of its query row's position",
                      (long long)(qsl[b] + i), (long long)slots[qsl[b] + i]);
    }
    std::vector<int64_t> written;
    for (int64_t t = 0; t < n_slots; ++t)
      if (slots[t] >= 0) written.push_back(slots[t]);
    std::sort(written.begin(), written.end());
    for (int64_t b = 0; b < B; ++b) {
      const int64_t older = seq_lens[b] - (qsl[b + 1] - qsl[b]);
      for (int64_t pos = 0; pos < older; ++pos)
        if (std::binary_search(written.begin(), written.end(), slot_of(b, pos)))
          return fail("sequence %lld reads slot %lld, which the step writes, at an older position", (long long)b,
                      (long long)slot_of(b, pos));
    }
  }
  return PKV_OK;
}

int paged_validate_metadata(const pkv_tensor* slot_mapping, const pkv_tensor* block_table,
                            const pkv_tensor* seq_lens, const pkv_tensor* query_start_loc,
                            int64_t num_pages, int64_t page_size, int64_t num_query_rows,
                            int64_t shared_prefix_pages, uint32_t checks, void* stream, char* message,
                            size_t message_len) {
  if (slot_mapping) PKV_TRY(check_tensor(slot_mapping, 1, 8));
  PKV_TRY(check_tensor(block_table, 2, 8));
  PKV_TRY(check_tensor(seq_lens, 1, 8));
  PKV_TRY(check_tensor(query_start_loc, 1, 8));
  if ((slot_mapping && slot_mapping->dtype != PKV_I64) || block_table->dtype != PKV_I64 ||
      seq_lens->dtype != PKV_I64 || query_start_loc->dtype != PKV_I64)
    return PKV_ERR_DTYPE;
  const int64_t B = block_table->shape[0];
  if (seq_lens->shape[0] != B || query_start_loc->shape[0] != B + 1) return PKV_ERR_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  auto fetch = [&](const pkv_tensor* t, std::vector<int64_t>& host) -> bool {
    host.resize((size_t)numel(t));
    if (host.empty()) return true;
    return hipMemcpyAsync(host.data(), t->data, host.size() * sizeof(int64_t), hipMemcpyDeviceToHost, s) ==
           hipSuccess;
  };
  std::vector<int64_t> sm, bt, sl, qs;
  if ((slot_mapping && !fetch(slot_mapping, sm)) || !fetch(block_table, bt) || !fetch(seq_lens, sl) ||
      !fetch(query_start_loc, qs))
    return PKV_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return PKV_ERR_HIP;
  return pkv_check_metadata_host(slot_mapping ? sm.data() : nullptr, (int64_t)sm.size(), bt.data(), B,
                                 block_table->shape[1], sl.data(), qs.data(), num_pages, page_size,
                                 num_query_rows, shared_prefix_pages, checks, message, message_len);
}

}  // extern "C"
