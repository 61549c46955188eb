// C ABI of the Block KV decode path: argument checks, the host-only entry
// points, and launches of the HIP kernels on the caller's stream.
// The contract of every function is documented in include/kvslot.h.
#include <limits.h>
#include <stdint.h>
#include <math.h>

#include "kvslot.h"
#include "kvslot_internal.h"

namespace {

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int launch_status(hipError_t e) { return e == hipSuccess ? KVS_OK : KVS_EHIP; }

// The kernels move element arrays with 16-byte vector operations and index
// arrays element by element: the former need 16-byte alignment, the latter
// their natural one. A null pointer counts as aligned (checked separately).
bool aligned(const void* ptr, uintptr_t a) { return ((uintptr_t)ptr & (a - 1)) == 0; }

int elem_bytes(kvs_dtype d) {
  switch (d) {
    case KVS_F32: return 4;
    case KVS_BF16: return 2;
    default: return 0;  // any other value, the range markers included: unsupported
  }
}

constexpr int kMaxRows = 64;        // (Hq / Hkv) * q_len: four MFMA column tiles of 16
constexpr int kMaxSeqs = kvs::kDecodeMaxSeqs;

}  // namespace

namespace {

// The step's tokens written by the decode launch itself (append entry point).
struct AppendArgs {
  const int32_t* req_indices;
  const int64_t* positions;
  int64_t num_tokens, max_num_tokens;
  int64_t* slot_mapping;
  const void* k_new;
  const void* v_new;
};

int decode_common(const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_table, int32_t table_stride, int32_t walk_blocks,
                  const int32_t* seq_lens, const int32_t* kv_pos_offset, int32_t window,
                  int32_t cp_world, int32_t cp_rank, int32_t cp_interleave,
                  int32_t num_seqs, int32_t q_len, int32_t num_q_heads, int32_t num_kv_heads,
                  int32_t head_dim, int32_t block_size, int64_t total_blocks, float scale,
                  kvs_dtype dtype, uint32_t flags, void* workspace, size_t workspace_bytes,
                  float* out, float* lse, void* stream, const AppendArgs* app = nullptr,
                  bool noalloc = false) {
  if (num_seqs < 0 || q_len < 1 || num_q_heads < 1 || num_kv_heads < 1 || head_dim < 1 ||
      block_size < 1 || table_stride < 1 || walk_blocks < 0 || walk_blocks > table_stride ||
      total_blocks < 1 || !isfinite(scale) || window < 0 || cp_world < 1 || cp_rank < 0 ||
      cp_rank >= cp_world || cp_interleave < 1)
    return KVS_EINVAL;
  if (!is_pow2(cp_interleave) || (block_size > 0 && block_size % cp_interleave != 0))
    return KVS_EINVAL;
  if (num_q_heads % num_kv_heads != 0) return KVS_EINVAL;
  if (flags & ~KVS_WALK_TABLE) return KVS_EINVAL;
  if (!elem_bytes(dtype)) return KVS_EUNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return KVS_EUNSUPPORTED;
  if (!is_pow2(block_size) || block_size < 16 || block_size > 256) return KVS_EUNSUPPORTED;
  if ((int64_t)(num_q_heads / num_kv_heads) * q_len > kMaxRows) return KVS_EUNSUPPORTED;
  if (num_seqs > kMaxSeqs) return KVS_EUNSUPPORTED;
  if ((int64_t)table_stride * block_size * cp_world > INT_MAX / 2) return KVS_EUNSUPPORTED;
  // the batch's 16-token tiles are counted in 32 bits, with headroom
  if ((int64_t)num_seqs * (walk_blocks * (int64_t)(block_size / 16) + 1) > INT_MAX / 2)
    return KVS_EUNSUPPORTED;
  if (app) {
    if (app->num_tokens < 0 || app->max_num_tokens < app->num_tokens) return KVS_EINVAL;
    if (app->max_num_tokens > 0 && !app->slot_mapping) return KVS_EINVAL;
    if (app->num_tokens > 0 && (!app->req_indices || !app->positions || !app->k_new ||
                                !app->v_new || !k_cache || !v_cache || !block_table))
      return KVS_EINVAL;
    if (!aligned(app->req_indices, 4) || !aligned(app->positions, 8) ||
        !aligned(app->slot_mapping, 8) || !aligned(app->k_new, 16) || !aligned(app->v_new, 16))
      return KVS_EINVAL;
    if (total_blocks > INT64_MAX / block_size) return KVS_EINVAL;
  }
  if (num_seqs == 0) {
    // no attention; the step's tokens are still written (no table row to hit)
    if (!app || app->max_num_tokens == 0) return KVS_OK;
    return launch_status(kvs::launch_slot_write(
        app->req_indices, app->positions, app->num_tokens, app->max_num_tokens, block_table, 0,
        table_stride, block_size, app->slot_mapping, app->k_new, app->v_new,
        const_cast<void*>(k_cache), const_cast<void*>(v_cache),
        total_blocks * block_size, num_kv_heads * head_dim * elem_bytes(dtype),
        (hipStream_t)stream));
  }
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !out || (!workspace && !noalloc))
    return KVS_EINVAL;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(kv_pos_offset, 4) ||
      !aligned(out, 16) || !aligned(lse, 4) || !aligned(workspace, 16))
    return KVS_EINVAL;
  // The caller's workspace must hold the size query's bound, which fits any
  // device; the library's own (noalloc) only what this launch uses.
  if (!noalloc && workspace_bytes < paged_decode_attention_workspace_bytes(
                                        num_seqs, q_len, num_q_heads, num_kv_heads, head_dim))
    return KVS_ENOSPACE;

  if (noalloc) {
    // the library's array on the current device, looked up on first use
    if (kvs::noalloc_scratch(&workspace) != hipSuccess) return KVS_EHIP;
    workspace_bytes = kvs::kNoallocScratchBytes;
  }
  kvs::DecodeParams p{};
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.kv_pos_offset = kv_pos_offset;
  p.out = out;
  p.lse_out = lse;
  p.chunk_meta = (int32_t*)workspace;
  p.partials = (float*)((char*)workspace + kvs::decode_meta_bytes(num_seqs));
  p.total_blocks = total_blocks;
  p.table_stride = table_stride;
  p.walk_blocks = walk_blocks;
  p.num_seqs = num_seqs;
  p.q_len = q_len;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.block_size = block_size;
  p.window = window;
  p.cp_world = cp_world;
  p.cp_rank = cp_rank;
  p.cp_ishift = __builtin_ctz((unsigned)cp_interleave);
  p.max_slices = kvs::decode_max_slices(num_kv_heads);
  p.min_tiles = 8;  // 128 tokens: partial traffic stays a few percent of the KV a slice reads
  // A segment start costs about three tile steps of streaming (measured
  // against two and four: three was the fastest or within 0.2% on the
  // 12-request, bucketing and 256-request batches).
  p.start_tiles = 3;
  p.scale_log2 = (float)((double)scale * 1.4426950408889634);  // log2(e)
  p.flags = flags;
  p.is_bf16 = dtype == KVS_BF16;
  if (app && app->max_num_tokens > 0) {
    p.app_req = app->req_indices;
    p.app_pos = app->positions;
    p.app_k = app->k_new;
    p.app_v = app->v_new;
    p.app_k_cache = const_cast<void*>(k_cache);
    p.app_v_cache = const_cast<void*>(v_cache);
    p.app_slots = app->slot_mapping;
    p.app_tokens = app->num_tokens;
    p.app_max_tokens = app->max_num_tokens;
  }
  if (noalloc) {
    // partial slots slice + request, below slices + num_seqs
    int slices = 0;
    if (kvs::decode_slices(p, &slices) != hipSuccess) return KVS_EHIP;
    const size_t need = kvs::decode_meta_bytes(num_seqs) +
                        kvs::decode_partial_slot_bytes(q_len, num_q_heads, head_dim) *
                            ((size_t)slices + (size_t)num_seqs);
    if (need > workspace_bytes) return KVS_ENOSPACE;
  }
  return launch_status(kvs::launch_paged_decode(p, (hipStream_t)stream));
}

}  // namespace

extern "C" {

const char* kvs_status_string(int status) {
  switch (status) {
    case KVS_OK: return "ok";
    case KVS_EINVAL: return "invalid argument";
    case KVS_EUNSUPPORTED: return "unsupported dtype, head_dim, block_size or shape";
    case KVS_EBUCKET: return "decode context-length bucket list fails validation";
    case KVS_ERANGE: return "needed_seq exceeds max_model_len";
    case KVS_ENOSPACE: return "workspace too small";
    case KVS_EHIP: return "HIP kernel launch failed";
  }
  return "unknown status";
}

int kv_slot_mapping(const int32_t* req_indices, const int64_t* positions, int64_t num_tokens,
                    int64_t max_num_tokens, const int32_t* block_table, int32_t table_rows,
                    int32_t table_stride, int32_t block_size, int64_t* slot_mapping,
                    void* stream) {
  if (num_tokens < 0 || max_num_tokens < num_tokens || table_rows < 0 || table_stride < 1 ||
      block_size < 1)
    return KVS_EINVAL;
  if (max_num_tokens > 0 && !slot_mapping) return KVS_EINVAL;
  if (num_tokens > 0 && (!req_indices || !positions)) return KVS_EINVAL;
  if (table_rows > 0 && !block_table) return KVS_EINVAL;
  if (!aligned(req_indices, 4) || !aligned(positions, 8) || !aligned(block_table, 4) ||
      !aligned(slot_mapping, 8))
    return KVS_EINVAL;
  return launch_status(kvs::launch_slot_mapping(req_indices, positions, num_tokens,
                                                max_num_tokens, block_table, table_rows,
                                                table_stride, block_size, slot_mapping,
                                                (hipStream_t)stream));
}

int kv_cache_write(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                   int64_t num_tokens, void* k_cache, void* v_cache, int64_t total_blocks,
                   int32_t block_size, int32_t num_kv_heads, int32_t head_dim, kvs_dtype dtype,
                   void* stream) {
  if (num_tokens < 0 || total_blocks < 1 || block_size < 1 || num_kv_heads < 1 || head_dim < 1)
    return KVS_EINVAL;
  const int es = elem_bytes(dtype);
  if (!es) return KVS_EUNSUPPORTED;
  const int64_t row_bytes = (int64_t)num_kv_heads * head_dim * es;
  if (row_bytes % 16 != 0 || row_bytes > INT_MAX) return KVS_EUNSUPPORTED;
  if (total_blocks > INT64_MAX / block_size) return KVS_EINVAL;
  if (num_tokens == 0) return KVS_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return KVS_EINVAL;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(slot_mapping, 8))
    return KVS_EINVAL;
  return launch_status(kvs::launch_cache_write(k_new, v_new, slot_mapping, num_tokens, k_cache,
                                               v_cache, total_blocks * block_size,
                                               (int32_t)row_bytes, (hipStream_t)stream));
}

int kv_slot_mapping_dcp(const int32_t* req_indices, const int64_t* positions, int64_t num_tokens,
                        int64_t max_num_tokens, const int32_t* block_table, int32_t table_rows,
                        int32_t table_stride, int32_t block_size, int32_t cp_world_size,
                        int32_t cp_rank, int32_t cp_interleave, int64_t* slot_mapping,
                        void* stream) {
  if (num_tokens < 0 || max_num_tokens < num_tokens || table_rows < 0 || table_stride < 1 ||
      block_size < 1 || cp_world_size < 1 || cp_rank < 0 || cp_rank >= cp_world_size ||
      cp_interleave < 1)
    return KVS_EINVAL;
  if (!is_pow2(block_size) || !is_pow2(cp_interleave) || block_size % cp_interleave != 0)
    return KVS_EINVAL;
  if (max_num_tokens > 0 && !slot_mapping) return KVS_EINVAL;
  if (num_tokens > 0 && (!req_indices || !positions)) return KVS_EINVAL;
  if (table_rows > 0 && !block_table) return KVS_EINVAL;
  if (!aligned(req_indices, 4) || !aligned(positions, 8) || !aligned(block_table, 4) ||
      !aligned(slot_mapping, 8))
    return KVS_EINVAL;
  return launch_status(kvs::launch_slot_mapping_dcp(
      req_indices, positions, num_tokens, max_num_tokens, block_table, table_rows, table_stride,
      block_size, cp_world_size, cp_rank, cp_interleave, slot_mapping, (hipStream_t)stream));
}

int kv_slot_mapping_cache_write(const int32_t* req_indices, const int64_t* positions,
                                int64_t num_tokens, int64_t max_num_tokens,
                                const int32_t* block_table, int32_t table_rows,
                                int32_t table_stride, int32_t block_size, int64_t* slot_mapping,
                                const void* k_new, const void* v_new, void* k_cache,
                                void* v_cache, int64_t total_blocks, int32_t num_kv_heads,
                                int32_t head_dim, kvs_dtype dtype, void* stream) {
  if (num_tokens < 0 || max_num_tokens < num_tokens || table_rows < 0 || table_stride < 1 ||
      block_size < 1 || total_blocks < 1 || num_kv_heads < 1 || head_dim < 1)
    return KVS_EINVAL;
  const int es = elem_bytes(dtype);
  if (!es) return KVS_EUNSUPPORTED;
  const int64_t row_bytes = (int64_t)num_kv_heads * head_dim * es;
  if (row_bytes % 16 != 0 || row_bytes > INT_MAX) return KVS_EUNSUPPORTED;
  if (total_blocks > INT64_MAX / block_size) return KVS_EINVAL;
  if (max_num_tokens > 0 && !slot_mapping) return KVS_EINVAL;
  if (num_tokens > 0 &&
      (!req_indices || !positions || !k_new || !v_new || !k_cache || !v_cache))
    return KVS_EINVAL;
  if (table_rows > 0 && !block_table) return KVS_EINVAL;
  if (!aligned(req_indices, 4) || !aligned(positions, 8) || !aligned(block_table, 4) ||
      !aligned(slot_mapping, 8) || !aligned(k_new, 16) || !aligned(v_new, 16) ||
      !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return KVS_EINVAL;
  return launch_status(kvs::launch_slot_write(
      req_indices, positions, num_tokens, max_num_tokens, block_table, table_rows, table_stride,
      block_size, slot_mapping, k_new, v_new, k_cache, v_cache, total_blocks * block_size,
      (int32_t)row_bytes, (hipStream_t)stream));
}

int select_ctx_bucket(int64_t max_num_computed_tokens, int32_t num_speculative_tokens,
                      const int32_t* buckets, int32_t num_buckets, int32_t max_model_len,
                      int32_t block_size, int32_t* bucket_len_out, int32_t* walk_blocks_out) {
  if (!bucket_len_out || !walk_blocks_out || num_buckets < 0 || max_num_computed_tokens < 0 ||
      num_speculative_tokens < 0 || max_model_len < 1 || block_size < 1)
    return KVS_EINVAL;
  const auto blocks_for = [&](int64_t len) { return (int32_t)((len + block_size - 1) / block_size); };
  if (!buckets) {  // feature off: the full table every step
    *bucket_len_out = max_model_len;
    *walk_blocks_out = blocks_for(max_model_len);
    return KVS_OK;
  }
  // "Validation": non-empty, positive, strictly ascending, below
  // max_model_len, divisible by P_MAX = 128.
  if (num_buckets == 0) return KVS_EBUCKET;
  for (int32_t i = 0; i < num_buckets; ++i) {
    const int32_t b = buckets[i];
    if (b <= 0 || b >= max_model_len || b % 128 != 0) return KVS_EBUCKET;
    if (i > 0 && b <= buckets[i - 1]) return KVS_EBUCKET;
  }
  // "Per-step bucket selection": needed_seq = max(num_computed_tokens) + 1 +
  // num_speculative_tokens; the smallest bucket >= needed_seq, falling back
  // to max_model_len.
  // (max_num_computed_tokens < max_model_len <= INT32_MAX keeps the sum in range)
  if (max_num_computed_tokens >= max_model_len) return KVS_ERANGE;
  const int64_t needed_seq = max_num_computed_tokens + 1 + (int64_t)num_speculative_tokens;
  if (needed_seq > max_model_len) return KVS_ERANGE;
  int32_t bucket = max_model_len;
  for (int32_t i = 0; i < num_buckets; ++i) {
    if (buckets[i] >= needed_seq) {
      bucket = buckets[i];  // ascending: the first that fits is the smallest
      break;
    }
  }
  *bucket_len_out = bucket;
  *walk_blocks_out = blocks_for(bucket);  // head trim: the first ceil(bucket / bs) blocks
  return KVS_OK;
}

int select_batch_bucket(int32_t num_active, const int32_t* buckets, int32_t num_buckets,
                        int32_t* padded_out) {
  if (!padded_out || num_active < 0 || num_buckets < 0) return KVS_EINVAL;
  if (num_buckets == 0 || !buckets) return KVS_EBUCKET;
  for (int32_t i = 0; i < num_buckets; ++i) {
    if (buckets[i] <= 0) return KVS_EBUCKET;
    if (i > 0 && buckets[i] <= buckets[i - 1]) return KVS_EBUCKET;
  }
  for (int32_t i = 0; i < num_buckets; ++i) {
    if (buckets[i] >= num_active) {  // ascending: the first that fits is the smallest
      *padded_out = buckets[i];
      return KVS_OK;
    }
  }
  return KVS_ERANGE;
}

int kv_map_to_kernel_blocks(const int32_t* src, int32_t rows, int32_t src_stride,
                            int32_t manager_block_size, int32_t kernel_block_size, int32_t* dst,
                            int32_t dst_stride) {
  if (rows < 0 || src_stride < 1 || manager_block_size < 1 || kernel_block_size < 1)
    return KVS_EINVAL;
  if (manager_block_size % kernel_block_size != 0) return KVS_EINVAL;
  const int32_t k = manager_block_size / kernel_block_size;
  if ((int64_t)src_stride * k > dst_stride) return KVS_EINVAL;
  if (rows == 0) return KVS_OK;
  if (!src || !dst) return KVS_EINVAL;
  for (int64_t r = 0; r < rows; ++r) {
    const int32_t* s = src + r * src_stride;
    int32_t* d = dst + r * dst_stride;
    for (int32_t c = 0; c < src_stride; ++c) {
      const int32_t m = s[c];
      for (int32_t i = 0; i < k; ++i) {
        if (m > 0) {
          const int64_t id = (int64_t)m * k + i;
          if (id > INT32_MAX) return KVS_EINVAL;
          d[(int64_t)c * k + i] = (int32_t)id;
        } else {
          d[(int64_t)c * k + i] = m;
        }
      }
    }
  }
  return KVS_OK;
}

size_t paged_decode_attention_workspace_bytes(int32_t num_seqs, int32_t q_len,
                                              int32_t num_q_heads, int32_t num_kv_heads,
                                              int32_t head_dim) {
  if (num_seqs < 0 || q_len < 1 || num_q_heads < 1 || num_kv_heads < 1 || head_dim < 1)
    return 0;
  return kvs::decode_meta_bytes(num_seqs) +
         kvs::decode_partial_bytes(num_seqs, q_len, num_q_heads, num_kv_heads, head_dim);
}

int paged_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_table, int32_t table_stride, int32_t walk_blocks,
                           const int32_t* seq_lens, int32_t num_seqs, int32_t q_len,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int64_t total_blocks, float scale,
                           kvs_dtype dtype, uint32_t flags, void* workspace,
                           size_t workspace_bytes, float* out, void* stream) {
  return decode_common(q, k_cache, v_cache, block_table, table_stride, walk_blocks, seq_lens,
                       nullptr, 0, 1, 0, 1, num_seqs, q_len, num_q_heads, num_kv_heads, head_dim,
                       block_size, total_blocks, scale, dtype, flags, workspace,
                       workspace_bytes, out, nullptr, stream);
}

int paged_decode_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, int32_t table_stride,
                                   int32_t walk_blocks, const int32_t* seq_lens, int32_t num_seqs,
                                   int32_t q_len, int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, int64_t total_blocks,
                                   float scale, kvs_dtype dtype, uint32_t flags, float* out,
                                   void* stream) {
  static_assert(KVS_NOALLOC_WORKSPACE_BYTES == kvs::kNoallocScratchBytes,
                "public and internal sizes of the library's workspace differ");
  return decode_common(q, k_cache, v_cache, block_table, table_stride, walk_blocks, seq_lens,
                       nullptr, 0, 1, 0, 1, num_seqs, q_len, num_q_heads, num_kv_heads, head_dim,
                       block_size, total_blocks, scale, dtype, flags, nullptr, 0, out, nullptr,
                       stream, nullptr, true);
}

int paged_decode_attention_swa(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, int32_t table_stride,
                               int32_t walk_blocks, const int32_t* seq_lens,
                               const int32_t* kv_pos_offset, int32_t sliding_window,
                               int32_t num_seqs, int32_t q_len, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int64_t total_blocks, float scale, kvs_dtype dtype,
                               void* workspace, size_t workspace_bytes, float* out,
                               void* stream) {
  return decode_common(q, k_cache, v_cache, block_table, table_stride, walk_blocks, seq_lens,
                       kv_pos_offset, sliding_window, 1, 0, 1, num_seqs, q_len, num_q_heads,
                       num_kv_heads, head_dim, block_size, total_blocks, scale, dtype, 0,
                       workspace, workspace_bytes, out, nullptr, stream);
}

int paged_decode_attention_dcp(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, int32_t table_stride,
                               int32_t walk_blocks, const int32_t* seq_lens, int32_t num_seqs,
                               int32_t q_len, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int64_t total_blocks,
                               float scale, kvs_dtype dtype, int32_t cp_world_size,
                               int32_t cp_rank, int32_t cp_interleave, void* workspace,
                               size_t workspace_bytes, float* out, float* lse, void* stream) {
  if (num_seqs > 0 && !lse) return KVS_EINVAL;
  return decode_common(q, k_cache, v_cache, block_table, table_stride, walk_blocks, seq_lens,
                       nullptr, 0, cp_world_size, cp_rank, cp_interleave, num_seqs, q_len,
                       num_q_heads, num_kv_heads, head_dim, block_size, total_blocks, scale,
                       dtype, 0, workspace, workspace_bytes, out, lse, stream);
}

int paged_decode_attention_append(const int32_t* req_indices, const int64_t* positions,
                                  int64_t num_tokens, int64_t max_num_tokens,
                                  int64_t* slot_mapping, const void* k_new, const void* v_new,
                                  const void* q, void* k_cache, void* v_cache,
                                  const int32_t* block_table, int32_t table_stride,
                                  int32_t walk_blocks, const int32_t* seq_lens, int32_t num_seqs,
                                  int32_t q_len, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, int64_t total_blocks,
                                  float scale, kvs_dtype dtype, uint32_t flags, void* workspace,
                                  size_t workspace_bytes, float* out, void* stream) {
  const AppendArgs app{req_indices, positions, num_tokens, max_num_tokens,
                       slot_mapping, k_new, v_new};
  return decode_common(q, k_cache, v_cache, block_table, table_stride, walk_blocks, seq_lens,
                       nullptr, 0, 1, 0, 1, num_seqs, q_len, num_q_heads, num_kv_heads, head_dim,
                       block_size, total_blocks, scale, dtype, flags, workspace,
                       workspace_bytes, out, nullptr, stream, &app);
}

int decode_lse_merge(const float* outs, const float* lses, int32_t world, int64_t rows,
                     int32_t head_dim, float* out, float* lse, void* stream) {
  if (world < 1 || rows < 0 || head_dim < 4 || head_dim % 4 != 0) return KVS_EINVAL;
  if (rows > 0 && (!outs || !lses || !out)) return KVS_EINVAL;
  if (!aligned(outs, 16) || !aligned(lses, 4) || !aligned(out, 16) || !aligned(lse, 4))
    return KVS_EINVAL;
  if (rows > INT64_MAX / head_dim / world) return KVS_EINVAL;
  return launch_status(
      kvs::launch_lse_merge(outs, lses, world, rows, head_dim, out, lse, (hipStream_t)stream));
}

int kv_swa_tail_trim(const int32_t* src, int32_t rows, int32_t src_stride,
                     const int32_t* seq_lens, int32_t q_len, int32_t sliding_window,
                     int32_t block_size, int32_t* dst, int32_t dst_stride, int32_t* kv_pos_offset,
                     int32_t* width_out) {
  if (rows < 0 || src_stride < 1 || q_len < 1 || sliding_window < 1 || block_size < 1 ||
      !width_out)
    return KVS_EINVAL;
  const int64_t need = ((int64_t)sliding_window + q_len - 1 + block_size - 1) / block_size + 1;
  const int32_t width = (int32_t)(need < src_stride ? need : src_stride);
  *width_out = width;
  if (dst_stride < width) return KVS_EINVAL;
  if (rows == 0) return KVS_OK;
  if (!src || !seq_lens || !dst || !kv_pos_offset) return KVS_EINVAL;
  for (int32_t r = 0; r < rows; ++r) {
    const int32_t L = seq_lens[r];
    const int64_t last = L > 0 ? (int64_t)(L - 1) / block_size : 0;
    const int64_t first = last - width + 1 > 0 ? last - width + 1 : 0;
    if (first * block_size > INT_MAX) return KVS_EINVAL;
    kv_pos_offset[r] = (int32_t)(first * block_size);
    for (int32_t c = 0; c < width; ++c) {
      const int64_t col = first + c;
      dst[(int64_t)r * dst_stride + c] = col < src_stride ? src[(int64_t)r * src_stride + col] : -1;
    }
  }
  return KVS_OK;
}

}  // extern "C"
