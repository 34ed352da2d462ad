// kernels.h -- internal launch interface between the C ABI layer and the
// gfx950 kernels.  Not part of the public ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedkv.h"

namespace pkv {

enum KvType { KV_F32 = 0, KV_BF16 = 1, KV_FP8 = 2 };

struct WriteParams {
  const void* k;
  const void* v;
  const int64_t* slots;
  void* key_pool;
  void* value_pool;
  int64_t n_tokens;
  int64_t row_bytes;  // Hkv * D * element size; a multiple of 16
};

// quantising form of the write: bf16 rows in, E4M3FN codes out
struct WriteFp8Params {
  const void* k;        // [n_tokens, Hkv, D] bf16
  const void* v;
  const int64_t* slots;
  void* key_pool;       // [num_pages, page_size, Hkv, D] E4M3FN codes
  void* value_pool;
  const float* k_scale;  // [Hkv] dequantisation factors
  const float* v_scale;
  int64_t n_tokens;
  int64_t Hkv, D;       // D a multiple of 8
};

struct AttnParams {
  const void* q;        // [T, Hq, D]
  void* out;            // [T, Hq, D]
  const void* key_pool;  // [num_pages, 16, Hkv, D]
  const void* value_pool;
  const int64_t* block_table;  // [B, max_blocks]
  const int64_t* seq_lens;     // [B]
  const int64_t* qsl;          // [B+1]
  const float* k_scale;        // [Hkv] (fp8 only)
  const float* v_scale;
  int64_t T, B, max_blocks, num_pages;
  int Hq, Hkv, D, G;
  float scale;
  int kv_type;         // KvType
  int max_query_len;   // grid sizing hint (>= true max n_b)
  // decode: stream-K over (sequence, 32-position block) units
  int split_tokens;    // requested positions per partition (0 = library choice)
  int grid_parts;      // partition ranges (parts) of the decode work, a multiple of the parts per workgroup
  int decode_rounds;   // consecutive parts each decode group runs as one stream (>= 1)
  int32_t* ws_cum;     // [B + 1] units before each sequence (written by workgroup 0)
  float* ws_ml;        // [B + grid_parts, Hq, 4] partial (max in log2 units, sum, unscale, unused)
  _Float16* ws_o;      // [B + grid_parts, Hq, D] unnormalised partial outputs times 1 / unscale
  // prefill work list: [0] item count, [1] tile count, then 2 words per item
  // (b << 16 | query tile, tile index * split_max_chunks + chunk), then the
  // (b << 16 | query tile) of every tile
  int32_t* ws_plan;
  int64_t plan_tiles_cap;  // bound on the (sequence, query tile) count
  // prefill key split (0 = off): an item's keys run as chunks of split_keys
  // keys (a multiple of 32), each writing (m, l, O) partials per row, which
  // prefill_split_merge_kernel combines
  int split_keys;
  int split_max_chunks;    // chunks an item may have (1 without the split)
  float* ws_split_ml;      // [plan_tiles_cap, Hkv, split_max_chunks, 256 rows, 4] (max, sum, unscale, unused)
  _Float16* ws_split_o;    // [plan_tiles_cap, Hkv, split_max_chunks, 256 rows, D] unnormalised rows / unscale
  // shared-prefix decode: the first prefix_len positions of every sequence
  // are the same pages; their attention runs as MFMA items of (prefix_tiles
  // groups of sequences) x (prefix_chunks chunks of prefix_chunk_len keys)
  int64_t prefix_len;  // 0 = off; a multiple of 32
  int prefix_tiles, prefix_chunks, prefix_chunk_len;
  // the prefix items run on prefix_wgs workgroups (a multiple of Hkv) beside
  // the decode grid, workgroup w taking items w / Hkv, w / Hkv + prefix_wgs /
  // Hkv, ... of KV head w % Hkv
  int prefix_wgs;
  float* ws_pre_ml;    // [prefix_chunks, B, Hq, 4] partial (max in log2 units, sum, unscale, unused)
  _Float16* ws_pre_o;  // [prefix_chunks, B, Hq, D] unnormalised partial outputs times 1 / unscale
  // decode fused with the write (n_new > 0, n_new = T: the new rows are the
  // query rows' own keys): decode_kernel takes the key at the last position
  // of the sequence owning query row t from row t of new_k/new_v [n_new, Hkv,
  // D] (pool dtype) instead of the pool, and writes each new row to its pool
  // row new_slots[t] (negative: skipped)
  const void* new_k;
  const void* new_v;
  const int64_t* new_slots;
  int64_t n_new;
  int kv_bytes;  // bytes per pool element (1 fp8, 2 bf16, 4 fp32)
};

// Optional events recorded around the main attention kernel of a launch.
struct LaunchEvents {
  hipEvent_t begin = nullptr;
  hipEvent_t end = nullptr;
};

hipError_t launch_write(const WriteParams& p, hipStream_t stream);
hipError_t launch_write_fp8(const WriteFp8Params& p, hipStream_t stream);
// (a shared-prefix decode, prefix_len > 0, runs its prefix items and the
// split-K pass as one launch of shared_prefix_decode_kernel, then the merge)
hipError_t launch_decode(const AttnParams& p, hipStream_t stream, const LaunchEvents& ev);
hipError_t launch_prefill(const AttnParams& p, hipStream_t stream, const LaunchEvents& ev);
hipError_t launch_attention_f32(const AttnParams& p, hipStream_t stream, const LaunchEvents& ev);
// the shared-prefix decode's split-K pass and prefix items as one launch
// (prefix_len > 0; the merge follows in launch_decode)
hipError_t launch_shared_prefix_decode(const AttnParams& p, hipStream_t stream);

hipError_t launch_csr_to_block_table(const int64_t* indptr, const int64_t* indices, const int64_t* last_len,
                                     int64_t nnz, int64_t B, int64_t max_blocks, int64_t page_size,
                                     int64_t pad_page, int64_t* block_table, int64_t* seq_lens,
                                     hipStream_t stream);

// workspace helpers shared by the ABI layer and the launchers.  The decode
// partial slots are sized for `parts` partition ranges: kDecodeMaxParts for a
// workspace that fits any device, or the grid's own count.
size_t decode_workspace_bytes(int64_t B, int Hq, int D, int parts);
// partition ranges of the decode work: a multiple of the parts one workgroup runs
int decode_grid_parts(int64_t B, int64_t max_len, int split_tokens, int n_cu, int Hkv);
// parts each group of a decode grid of one workgroup per CU (n_cu of them) runs:
// grid_parts / (groups * n_cu) when that divides evenly, else 1 (a workgroup per
// part)
int decode_rounds(int grid_parts, int n_cu, int Hkv);
// whether the decode launch planned in p (grid_parts set) can also write
// n_new rows of row_bytes each (the fused write)
bool decode_can_fuse_write(const AttnParams& p, int64_t n_new, int64_t row_bytes);
void decode_workspace_carve(AttnParams& p, void* workspace, int parts);
constexpr int kDecodeMaxParts = 2048;
constexpr int kDecodeMaxSeqs = 4096;
// decides the prefill key split (fills plan_tiles_cap, split_keys,
// split_max_chunks); then the workspace size and its carving
void prefill_split_plan(AttnParams& p);
size_t prefill_workspace_bytes(const AttnParams& p);
void prefill_workspace_carve(AttnParams& p, void* workspace);
constexpr int kMaxPrefixChunks = 8;
// prefill workgroups one launch may hold (512 threads each: 2^31 work-items,
// below the launch limit of 2^32)
constexpr int64_t kPrefillMaxGroups = (int64_t)1 << 22;
// groups of decode sequences, chunks and chunk length of a shared prefix of
// prefix_len positions, and the workgroups its items run on beside the
// decode, a share of the n_cu CUs (fills p.prefix_*; n_cu = 0 when the device
// is not known).  Returns the partials' workspace bytes: for the planned
// chunks when `tight`, else for the most chunks any plan can choose,
// min(kMaxPrefixChunks, prefix_len / 32) (a size that fits any device).
size_t prefix_plan(AttnParams& p, int64_t prefix_len, int n_cu, bool tight);
void prefix_workspace_carve(AttnParams& p, void* region);
int prefill_tokens_per_tile(int G);

// paged_attention whose workspace is a fixed region of region_bytes bytes on
// each device, resolved by region(device) once the call is known to fit
// (PKV_ERR_SCRATCH otherwise); decode partials are sized for the device's own
// grid.  Implemented by the ABI layer.
int attention_in_region(const pkv_tensor* q, const pkv_tensor* key_pool, const pkv_tensor* value_pool,
                        const pkv_tensor* block_table, const pkv_tensor* seq_lens,
                        const pkv_tensor* query_start_loc, float scale, pkv_tensor* out,
                        const pkv_attn_opts* opts, size_t region_bytes, void* (*region)(int device),
                        void* stream);
int64_t prefill_max_items(int64_t T, int64_t B, int G);

}  // namespace pkv
