/*
 * pagedkv_oracle.c -- plain CPU oracle for the paged KV write and paged
 * attention step.
 *
 * THIS IS TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it.  The GPU library never links,
 * includes or calls anything in this file, and this file includes nothing
 * from the GPU library.
 *
 * What it computes is the plain definition of the step, written out the slow
 * and obvious way, in fp64:
 *
 *   1. write:   every new token's K and V row is copied byte for byte into the
 *               page pool at the row named by its slot (for fp8 pools a
 *               second form encodes bf16 rows into E4M3FN codes on the way)
 *               (page "Add paged / block-table KV cache export
 *               (--features paged-cache)", onnxruntime/mobius #395, PR summary
 *               and table "ONNX I/O contract": slot = page_id*page_size+offset,
 *               pools are [num_pages, page_size, kv_hidden], written with
 *               ScatterND).
 *   2. gather:  each sequence's pages are assembled into a contiguous cache by
 *               following its block_table row page by page (same page, PR
 *               summary: Gather(pool, block_table)).
 *   3. attend:  causal GQA softmax attention whose key range is cut to
 *               nonpad_kv_seqlen, the total valid length after the write
 *               (same page, "How it works" step 3 and the I/O contract table:
 *               opset-24 Attention with is_causal=1 and nonpad_kv_seqlen).
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - the new tokens of a sequence are its last n_b positions, so query i of
 *     sequence b sits at position L_b - n_b + i and sees keys 0..that position
 *     (bottom-right causal alignment);
 *   - query head hq reads KV head hq / G with G = Hq / Hkv, so consecutive
 *     query heads share a KV head (page "[Draft] kv paged kernels",
 *     ROCm/maxtext #93, the kv_pool_sharding commit maps each query head to a
 *     KV head by integer division by the replication factor);
 *   - kv_hidden is head-major: head h occupies elements [h*D, (h+1)*D);
 *   - a negative slot means "no write";
 *   - duplicate non-negative slots in one call are rejected;
 *   - fp8 pools hold OCP E4M3FN codes with one fp32 scale per KV head per pool;
 *   - the quantising write encodes x / scale[h] (one binary32 division) by
 *     round to nearest even, saturating at +-448;
 *   - scale multiplies q.k exactly as passed, with no implicit 1/sqrt(D)
 *     (maxtext #93, gpu_paged commit and the scale-fix commit: the caller owns
 *     the scale).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_ERR_SLOT_RANGE (-1)
#define ORC_ERR_SLOT_DUPLICATE (-2)
#define ORC_ERR_PAGE_ID (-3)
#define ORC_ERR_METADATA (-4)
#define ORC_ERR_DTYPE (-5)
#define ORC_ERR_NOMEM (-6)

/* element type codes shared with the Python wrapper of this oracle */
#define ORC_F32 0
#define ORC_BF16 1
#define ORC_FP8_E4M3FN 2

static int64_t elem_size(int dtype) {
  switch (dtype) {
    case ORC_F32: return 4;
    case ORC_BF16: return 2;
    case ORC_FP8_E4M3FN: return 1;
    default: return 0;
  }
}

/* bfloat16 is the top half of an IEEE binary32: widen by shifting the 16 bits
 * into the high half of a 32-bit word. */
double orc_bf16_to_double(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP 8-bit E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.
 * Exponent field 0 encodes subnormals m/8 * 2^-6; the all-ones pattern
 * S.1111.111 is NaN; there are no infinities, so S.1111.110 = +-448 is the
 * largest finite value. */
double orc_e4m3fn_to_double(uint8_t code) {
  int sign = (code >> 7) & 1;
  int exponent = (code >> 3) & 0xF;
  int mantissa = code & 0x7;
  double magnitude;
  if (exponent == 0xF && mantissa == 0x7) return NAN;
  if (exponent == 0)
    magnitude = ldexp((double)mantissa / 8.0, 1 - 7);
  else
    magnitude = ldexp(1.0 + (double)mantissa / 8.0, exponent - 7);
  return sign ? -magnitude : magnitude;
}

void orc_e4m3fn_table(double out[256]) {
  for (int c = 0; c < 256; ++c) out[c] = orc_e4m3fn_to_double((uint8_t)c);
}

/* One element of a KV pool or query tensor, widened to fp64.  For fp8 the
 * per-KV-head scale multiplies the decoded code; the product of a 4-bit and a
 * 24-bit significand is exact in fp64. */
static double load_elem(const void* base, int dtype, int64_t index, double fp8_scale) {
  switch (dtype) {
    case ORC_F32: return (double)((const float*)base)[index];
    case ORC_BF16: return orc_bf16_to_double(((const uint16_t*)base)[index]);
    case ORC_FP8_E4M3FN: return orc_e4m3fn_to_double(((const uint8_t*)base)[index]) * fp8_scale;
    default: return NAN;
  }
}

/*
 * Step 1: the write.  k and v are [n_tokens, row_bytes] byte rows (one row is
 * Hkv*D elements of the pool dtype); the pools are [num_pages, page_size,
 * row_bytes].  Rows are copied unchanged, so NaN payloads survive.
 */
int orc_paged_kv_write(const uint8_t* k, const uint8_t* v, const int64_t* slot_mapping,
                       int64_t n_tokens, uint8_t* key_pool, uint8_t* value_pool,
                       int64_t num_pages, int64_t page_size, int64_t row_bytes) {
  int64_t capacity = num_pages * page_size;
  /* validate everything before touching the pools */
  for (int64_t t = 0; t < n_tokens; ++t) {
    int64_t s = slot_mapping[t];
    if (s < 0) continue;
    if (s >= capacity) return ORC_ERR_SLOT_RANGE;
    for (int64_t u = 0; u < t; ++u)
      if (slot_mapping[u] == s) return ORC_ERR_SLOT_DUPLICATE;
  }
  for (int64_t t = 0; t < n_tokens; ++t) {
    int64_t s = slot_mapping[t];
    if (s < 0) continue;
    int64_t page = s / page_size;
    int64_t offset = s % page_size;
    int64_t dst_row = page * page_size + offset;
    memcpy(key_pool + dst_row * row_bytes, k + t * row_bytes, (size_t)row_bytes);
    memcpy(value_pool + dst_row * row_bytes, v + t * row_bytes, (size_t)row_bytes);
  }
  return ORC_OK;
}

/* E4M3FN encoding of a binary32 value y: the finite code nearest to y, a
 * tie going to the code whose mantissa LSB is 0 (round to nearest even), and
 * magnitudes beyond the largest finite value (infinities included) going to
 * +-448 (saturation: the format has no infinity).  NaN gives the NaN code
 * with y's sign; the sign of zero is kept.  Found by plain search over the
 * 127 non-negative finite codes. */
uint8_t orc_e4m3fn_from_float(float y) {
  uint8_t sign = signbit(y) ? 0x80 : 0x00;
  if (isnan(y)) return sign | 0x7F;
  double a = fabs((double)y);
  if (isinf(a)) return sign | 0x7E;
  int best = 0;
  double best_d = a; /* distance to code 0 (+0) */
  for (int c = 1; c <= 0x7E; ++c) {
    double d = fabs(orc_e4m3fn_to_double((uint8_t)c) - a);
    if (d < best_d || (d == best_d && (c & 1) == 0)) {
      best = c;
      best_d = d;
    }
  }
  return sign | (uint8_t)best;
}

void orc_e4m3fn_encode_array(const float* y, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3fn_from_float(y[i]);
}

/*
 * Step 1 for fp8 pools, with the quantisation folded into the write: k and v
 * are bf16 rows [n_tokens, Hkv, D]; element x of KV head h is stored as the
 * E4M3FN code of x / scale[h], the quotient taken once in binary32 (the
 * scales are the per-head dequantisation factors the attention multiplies
 * codes by); a NaN input is stored as the NaN code with its own sign.
 * Slots are checked and skipped exactly as in the plain write.
 */
int orc_paged_kv_write_fp8(const uint16_t* k, const uint16_t* v, const int64_t* slot_mapping,
                           int64_t n_tokens, const float* k_scale, const float* v_scale,
                           uint8_t* key_pool, uint8_t* value_pool, int64_t num_pages,
                           int64_t page_size, int64_t Hkv, int64_t D) {
  int64_t capacity = num_pages * page_size;
  int64_t row = Hkv * D;
  for (int64_t t = 0; t < n_tokens; ++t) {
    int64_t s = slot_mapping[t];
    if (s < 0) continue;
    if (s >= capacity) return ORC_ERR_SLOT_RANGE;
    for (int64_t u = 0; u < t; ++u)
      if (slot_mapping[u] == s) return ORC_ERR_SLOT_DUPLICATE;
  }
  for (int64_t t = 0; t < n_tokens; ++t) {
    int64_t s = slot_mapping[t];
    if (s < 0) continue;
    int64_t dst_row = (s / page_size) * page_size + s % page_size;
    for (int64_t h = 0; h < Hkv; ++h)
      for (int64_t i = 0; i < D; ++i) {
        int64_t e = h * D + i;
        float xk = (float)orc_bf16_to_double(k[t * row + e]);
        float xv = (float)orc_bf16_to_double(v[t * row + e]);
        /* a NaN input keeps its own sign (a quotient's NaN sign is not fixed by IEEE 754) */
        key_pool[dst_row * row + e] =
            isnan(xk) ? (uint8_t)(signbit(xk) ? 0xFF : 0x7F) : orc_e4m3fn_from_float(xk / k_scale[h]);
        value_pool[dst_row * row + e] =
            isnan(xv) ? (uint8_t)(signbit(xv) ? 0xFF : 0x7F) : orc_e4m3fn_from_float(xv / v_scale[h]);
      }
  }
  return ORC_OK;
}

/*
 * The packed (CSR) page-list form of the metadata, unpacked into the
 * row-padded block table: sequence b's pages are
 * indices[indptr[b] .. indptr[b+1]) and its last page holds last_len[b] rows
 * (page "Refactor KV Cache Manager with a new torch exportable KVCache
 * backend", NVIDIA/recsys-examples #400, the KVCacheMetadata fields
 * kv_indices, kv_indptr, kv_last_page_len).  Rows are padded with pad_page;
 * a sequence with no page has length 0.  Inconsistent metadata (indptr
 * decreasing or past nnz, more than max_blocks pages, a last-page length
 * outside 1..page_size) is rejected.
 */
int orc_block_table_from_csr(const int64_t* indptr, const int64_t* indices, int64_t nnz, const int64_t* last_len,
                             int64_t B, int64_t page_size, int64_t pad_page, int64_t max_blocks,
                             int64_t* block_table, int64_t* seq_lens) {
  if (indptr[0] != 0) return ORC_ERR_METADATA;
  for (int64_t b = 0; b < B; ++b) {
    int64_t n = indptr[b + 1] - indptr[b];
    if (n < 0 || indptr[b + 1] > nnz || n > max_blocks) return ORC_ERR_METADATA;
    if (n > 0 && (last_len[b] < 1 || last_len[b] > page_size)) return ORC_ERR_METADATA;
  }
  for (int64_t b = 0; b < B; ++b) {
    int64_t n = indptr[b + 1] - indptr[b];
    for (int64_t j = 0; j < max_blocks; ++j)
      block_table[b * max_blocks + j] = j < n ? indices[indptr[b] + j] : pad_page;
    seq_lens[b] = n > 0 ? (n - 1) * page_size + last_len[b] : 0;
  }
  return ORC_OK;
}

/*
 * Steps 2 and 3: gather and attend.
 *
 *   q                [T, Hq, D]            q_dtype (f32 or bf16)
 *   key/value_pool   [num_pages, page_size, Hkv, D]   kv_dtype
 *   k_scale/v_scale  [Hkv] fp32, only read for fp8 pools
 *   block_table      [B, max_blocks] i64
 *   seq_lens         [B] i64   total valid KV length after the write
 *   query_start_loc  [B+1] i64 packed query rows of sequence b are
 *                    query_start_loc[b] .. query_start_loc[b+1]-1
 *   sel_tokens       which packed query rows to compute (NULL = all T rows)
 *   out              [n_sel, Hq, D] fp64
 */
int orc_paged_attention(const void* q, int q_dtype, int64_t T, int64_t Hq,
                        const void* key_pool, const void* value_pool, int kv_dtype,
                        int64_t num_pages, int64_t page_size, int64_t Hkv, int64_t D,
                        const float* k_scale, const float* v_scale,
                        const int64_t* block_table, int64_t B, int64_t max_blocks,
                        const int64_t* seq_lens, const int64_t* query_start_loc,
                        double scale, const int64_t* sel_tokens, int64_t n_sel,
                        double* out, int n_threads) {
  if (elem_size(kv_dtype) == 0 || (q_dtype != ORC_F32 && q_dtype != ORC_BF16))
    return ORC_ERR_DTYPE;
  if (kv_dtype == ORC_FP8_E4M3FN && (k_scale == NULL || v_scale == NULL))
    return ORC_ERR_DTYPE;
  if (Hkv <= 0 || Hq % Hkv != 0) return ORC_ERR_METADATA;
  const int64_t G = Hq / Hkv;
  if (sel_tokens == NULL) n_sel = T;

  /* metadata checks: ordered query spans that end at T, n_b <= L_b, and the
   * table is wide enough for every length */
  if (query_start_loc[0] != 0 || query_start_loc[B] != T) return ORC_ERR_METADATA;
  for (int64_t b = 0; b < B; ++b) {
    int64_t n_b = query_start_loc[b + 1] - query_start_loc[b];
    if (n_b < 0 || n_b > seq_lens[b]) return ORC_ERR_METADATA;
    if (seq_lens[b] > max_blocks * page_size) return ORC_ERR_METADATA;
  }
  for (int64_t s = 0; s < n_sel; ++s) {
    int64_t t = sel_tokens ? sel_tokens[s] : s;
    if (t < 0 || t >= T) return ORC_ERR_METADATA;
  }
  /* every block_table entry that a sequence's length reaches must name a page */
  for (int64_t b = 0; b < B; ++b) {
    int64_t n_blocks = (seq_lens[b] + page_size - 1) / page_size;
    for (int64_t j = 0; j < n_blocks; ++j) {
      int64_t page = block_table[b * max_blocks + j];
      if (page < 0 || page >= num_pages) return ORC_ERR_PAGE_ID;
    }
  }

  const double one = 1.0;
  int status = ORC_OK;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bh = 0; bh < B * Hkv; ++bh) {
    const int64_t b = bh / Hkv;
    const int64_t h = bh % Hkv;
    const int64_t L = seq_lens[b];
    const int64_t q_begin = query_start_loc[b];
    const int64_t n_b = query_start_loc[b + 1] - q_begin;

    /* does this sequence own any selected row? */
    int any = 0;
    for (int64_t s = 0; s < n_sel && !any; ++s) {
      int64_t t = sel_tokens ? sel_tokens[s] : s;
      if (t >= q_begin && t < q_begin + n_b) any = 1;
    }
    if (!any || L == 0) continue;

    /* step 2: gather this head's K and V rows, page by page */
    double* Kc = (double*)malloc((size_t)(L * D) * sizeof(double));
    double* Vc = (double*)malloc((size_t)(L * D) * sizeof(double));
    double* x = (double*)malloc((size_t)L * sizeof(double));
    double* qv = (double*)malloc((size_t)D * sizeof(double));
    if (!Kc || !Vc || !x || !qv) {
#pragma omp atomic write
      status = ORC_ERR_NOMEM;
      free(Kc); free(Vc); free(x); free(qv);
      continue;
    }
    const double ks = kv_dtype == ORC_FP8_E4M3FN ? (double)k_scale[h] : one;
    const double vs = kv_dtype == ORC_FP8_E4M3FN ? (double)v_scale[h] : one;
    const int64_t n_blocks = (L + page_size - 1) / page_size;
    for (int64_t j = 0; j < n_blocks; ++j) {
      const int64_t page = block_table[b * max_blocks + j];
      for (int64_t o = 0; o < page_size; ++o) {
        const int64_t pos = j * page_size + o;
        if (pos >= L) break;
        const int64_t base = ((page * page_size + o) * Hkv + h) * D;
        for (int64_t d = 0; d < D; ++d) {
          Kc[pos * D + d] = load_elem(key_pool, kv_dtype, base + d, ks);
          Vc[pos * D + d] = load_elem(value_pool, kv_dtype, base + d, vs);
        }
      }
    }

    /* step 3: two-pass softmax attention for every selected row of b */
    for (int64_t s = 0; s < n_sel; ++s) {
      const int64_t t = sel_tokens ? sel_tokens[s] : s;
      if (t < q_begin || t >= q_begin + n_b) continue;
      const int64_t i = t - q_begin;
      const int64_t p = L - n_b + i; /* absolute position of this query row */
      for (int64_t hq = h * G; hq < (h + 1) * G; ++hq) {
        for (int64_t d = 0; d < D; ++d)
          qv[d] = load_elem(q, q_dtype, (t * Hq + hq) * D + d, one);
        double m = -INFINITY;
        for (int64_t u = 0; u <= p; ++u) {
          double dot = 0.0;
          for (int64_t d = 0; d < D; ++d) dot += qv[d] * Kc[u * D + d];
          x[u] = scale * dot;
          if (x[u] > m) m = x[u];
        }
        double denom = 0.0;
        for (int64_t u = 0; u <= p; ++u) {
          x[u] = exp(x[u] - m);
          denom += x[u];
        }
        double* o_row = out + (s * Hq + hq) * D;
        for (int64_t d = 0; d < D; ++d) {
          double acc = 0.0;
          for (int64_t u = 0; u <= p; ++u) acc += x[u] * Vc[u * D + d];
          o_row[d] = acc / denom;
        }
      }
    }
    free(Kc); free(Vc); free(x); free(qv);
  }
  return status;
}

int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
