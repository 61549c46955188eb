// Host-side memory and undefined-behaviour check of the C ABI's host logic.
//
// tests/test_host_sanitize.py builds this driver and the library sources with
// AddressSanitizer and UBSan on the host code only (no kernel is launched
// here) and runs it. Every array the
// library reads or writes is a heap allocation of exactly the size the call
// is entitled to touch, so a read or write past it stops the run. The
// results are checked against the rules the header states; the exact values
// are pinned against the oracle elsewhere (test_abi_host.py).
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "kvslot.h"

namespace {

int g_checks = 0;

void require(bool ok, const char* what, long a = 0, long b = 0) {
  ++g_checks;
  if (!ok) {
    std::fprintf(stderr, "FAILED: %s (%ld, %ld)\n", what, a, b);
    std::exit(1);
  }
}

// Exactly-sized heap copy (std::vector of that size; no spare capacity used).
std::vector<int32_t> exact(const std::vector<int32_t>& v) { return std::vector<int32_t>(v); }

void check_select_ctx_bucket() {
  const std::vector<std::vector<int32_t>> lists = {
      {128}, {128, 256}, {256, 128}, {100}, {0}, {-128}, {4096}, {4096, 8192, 16384},
      {128, 128}, {384, 512, 1024, 2048}};
  const int32_t mmls[] = {128, 512, 4096, 131072};
  const int32_t bss[] = {1, 16, 64, 256};
  for (int32_t mml : mmls)
    for (int32_t bs : bss)
      for (int spec = 0; spec <= 3; ++spec)
        for (int64_t ctx = 0; ctx <= 600; ctx += 7) {
          int32_t b = -1, w = -1;
          int st = select_ctx_bucket(ctx, spec, nullptr, 0, mml, bs, &b, &w);
          if (ctx + 1 + spec <= mml) {
            require(st == KVS_OK && b == mml && w == (mml + bs - 1) / bs, "feature off", ctx, st);
          } else {
            require(st == KVS_ERANGE || st == KVS_OK, "feature off status", ctx, st);
          }
          for (const auto& l : lists) {
            std::vector<int32_t> buf = exact(l);
            st = select_ctx_bucket(ctx, spec, buf.data(), (int32_t)buf.size(), mml, bs, &b, &w);
            require(st == KVS_OK || st == KVS_EBUCKET || st == KVS_ERANGE, "status", ctx, st);
            if (st == KVS_OK) {
              const int64_t need = ctx + 1 + spec;
              require(b >= need && b <= mml, "bucket covers needed_seq", b, need);
              require(w == (b + bs - 1) / bs, "walk = ceil(bucket / bs)", w, b);
            }
          }
          // empty non-null list: invalid
          std::vector<int32_t> one(1, 128);
          st = select_ctx_bucket(ctx, spec, one.data(), 0, mml, bs, &b, &w);
          require(st == KVS_EBUCKET, "empty list", ctx, st);
        }
  int32_t b, w;
  require(select_ctx_bucket(-1, 0, nullptr, 0, 4096, 64, &b, &w) == KVS_EINVAL, "negative ctx");
  require(select_ctx_bucket(0, -1, nullptr, 0, 4096, 64, &b, &w) == KVS_EINVAL, "negative spec");
  require(select_ctx_bucket(0, 0, nullptr, 0, 0, 64, &b, &w) == KVS_EINVAL, "mml 0");
  require(select_ctx_bucket(0, 0, nullptr, 0, 4096, 0, &b, &w) == KVS_EINVAL, "bs 0");
  require(select_ctx_bucket(0, 0, nullptr, 0, 4096, 64, nullptr, &w) == KVS_EINVAL, "null out");
  std::vector<int32_t> l128 = {128};
  require(select_ctx_bucket(INT64_MAX, INT32_MAX, l128.data(), 1, 4096, 64, &b, &w) == KVS_ERANGE,
          "huge needed_seq");
  require(select_ctx_bucket(4095, INT32_MAX, l128.data(), 1, 4096, 64, &b, &w) == KVS_ERANGE,
          "huge speculative count");
  require(select_ctx_bucket(INT64_MAX, INT32_MAX, nullptr, 0, 4096, 64, &b, &w) == KVS_OK &&
              b == 4096 && w == 64,
          "feature off ignores needed_seq");
  require(select_ctx_bucket(0, 0, nullptr, 0, INT32_MAX, 1, &b, &w) == KVS_OK && w == INT32_MAX,
          "walk at INT32_MAX");
}

void check_select_batch_bucket(std::mt19937& rng) {
  for (int it = 0; it < 2000; ++it) {
    const int n = (int)(rng() % 6);
    std::vector<int32_t> l(n);
    int32_t v = (int32_t)(rng() % 4) - 1;
    for (int i = 0; i < n; ++i) {
      v += (int32_t)(rng() % 9) - 1;
      l[i] = v;
    }
    const int32_t active = (int32_t)(rng() % 40) - 2;
    int32_t out = -7;
    const int st = select_batch_bucket(active, n ? l.data() : nullptr, n, &out);
    require(st == KVS_OK || st == KVS_EINVAL || st == KVS_EBUCKET || st == KVS_ERANGE,
            "batch bucket status", st);
    if (st == KVS_OK) {
      bool found = false;
      for (int i = 0; i < n; ++i) found |= l[i] == out;
      require(found && out >= active, "batch bucket fits", out, active);
    }
  }
  int32_t out;
  require(select_batch_bucket(1, nullptr, 0, &out) == KVS_EBUCKET, "no buckets");
  std::vector<int32_t> l = {1, 2, 4};
  require(select_batch_bucket(3, l.data(), 3, nullptr) == KVS_EINVAL, "null out");
  require(select_batch_bucket(5, l.data(), 3, &out) == KVS_ERANGE, "too many requests");
}

void check_map_to_kernel_blocks(std::mt19937& rng) {
  const int32_t mbs[] = {16, 32, 64, 128};
  const int32_t kbs[] = {1, 8, 16, 32, 48};
  for (int it = 0; it < 600; ++it) {
    const int32_t rows = (int32_t)(rng() % 5);
    const int32_t ss = 1 + (int32_t)(rng() % 7);
    const int32_t m = mbs[rng() % 4], kb = kbs[rng() % 5];
    const int32_t k = (kb > 0 && m % kb == 0) ? m / kb : 1;
    const int32_t ds = ss * k + (int32_t)(rng() % 3) - 1;  // sometimes one short
    std::vector<int32_t> src((size_t)rows * ss);
    for (auto& e : src) e = (int32_t)(rng() % 5) == 0 ? -1 : (int32_t)(rng() % 1000);
    std::vector<int32_t> dst((size_t)rows * (ds > 0 ? ds : 0), 12345);
    const int st = kv_map_to_kernel_blocks(rows ? src.data() : nullptr, rows, ss, m, kb,
                                           rows ? dst.data() : nullptr, ds);
    const bool valid = m % kb == 0 && ds >= ss * k;
    if (rows == 0) {
      require(st == KVS_OK || st == KVS_EINVAL, "empty table", st);
      continue;
    }
    require(valid ? st == KVS_OK : st == KVS_EINVAL, "expansion status", st, valid);
    if (st != KVS_OK) continue;
    for (int32_t r = 0; r < rows; ++r)
      for (int32_t c = 0; c < ss; ++c)
        for (int32_t i = 0; i < k; ++i) {
          const int32_t e = src[(size_t)r * ss + c];
          const int32_t want = e > 0 ? e * k + i : e;
          require(dst[(size_t)r * ds + c * k + i] == want, "expanded entry", e, i);
        }
  }
  // an id whose expansion leaves int32 is rejected, not wrapped
  std::vector<int32_t> src = {INT32_MAX / 2};
  std::vector<int32_t> dst(4);
  require(kv_map_to_kernel_blocks(src.data(), 1, 1, 64, 16, dst.data(), 4) == KVS_EINVAL,
          "expanded id beyond int32");
}

void check_swa_tail_trim(std::mt19937& rng) {
  for (int it = 0; it < 600; ++it) {
    const int32_t rows = 1 + (int32_t)(rng() % 4);
    const int32_t ss = 1 + (int32_t)(rng() % 40);
    const int32_t bs = 1 << (rng() % 7);
    const int32_t q_len = 1 + (int32_t)(rng() % 4);
    const int32_t window = 1 + (int32_t)(rng() % 300);
    std::vector<int32_t> src((size_t)rows * ss);
    for (auto& e : src) e = (int32_t)(rng() % 50);
    std::vector<int32_t> lens(rows);
    for (auto& L : lens) L = (int32_t)(rng() % (ss * bs + 1));
    // first call with room for nothing: reports the width
    std::vector<int32_t> off(rows);
    int32_t width = -1;
    std::vector<int32_t> none(1);
    int st = kv_swa_tail_trim(src.data(), rows, ss, lens.data(), q_len, window, bs, none.data(), 0,
                              off.data(), &width);
    require(width >= 1 && width <= ss, "reported width", width, ss);
    require(st == KVS_EINVAL, "short destination rejected", st);
    std::vector<int32_t> dst((size_t)rows * width);
    st = kv_swa_tail_trim(src.data(), rows, ss, lens.data(), q_len, window, bs, dst.data(), width,
                          off.data(), &width);
    require(st == KVS_OK, "trim status", st);
    for (int32_t r = 0; r < rows; ++r) {
      require(off[r] >= 0 && off[r] % bs == 0, "offset is a block start", off[r], bs);
      const int32_t c0 = off[r] / bs;
      for (int32_t c = 0; c < width; ++c) {
        const int32_t got = dst[(size_t)r * width + c];
        const int32_t want = c0 + c < ss ? src[(size_t)r * ss + c0 + c] : got;
        require(got == want, "trimmed column copies the table", got, want);
      }
    }
  }
}

void check_gpu_entry_argument_checks() {
  // Invalid scalars and null pointers: every GPU entry returns before any
  // device work (no pointer here is dereferenced).
  require(kv_slot_mapping(nullptr, nullptr, -1, 0, nullptr, 0, 1, 16, nullptr, nullptr) == KVS_EINVAL,
          "slot mapping negative count");
  require(kv_slot_mapping(nullptr, nullptr, 4, 2, nullptr, 0, 1, 16, nullptr, nullptr) == KVS_EINVAL,
          "slot mapping max < count");
  require(kv_slot_mapping(nullptr, nullptr, 0, 0, nullptr, 0, 1, 16, nullptr, nullptr) == KVS_OK,
          "slot mapping with nothing to do");
  require(kv_cache_write(nullptr, nullptr, nullptr, -1, nullptr, nullptr, 1, 16, 8, 128, KVS_BF16,
                         nullptr) == KVS_EINVAL,
          "cache write negative count");
  require(kv_cache_write(nullptr, nullptr, nullptr, 0, nullptr, nullptr, 1, 16, 8, 128, (kvs_dtype)7,
                         nullptr) == KVS_EUNSUPPORTED,
          "cache write dtype");
  require(kv_cache_write(nullptr, nullptr, nullptr, 0, nullptr, nullptr, 1, 16, 8, 128, (kvs_dtype)-3,
                         nullptr) == KVS_EUNSUPPORTED,
          "cache write negative dtype");
  const int st = paged_decode_attention(nullptr, nullptr, nullptr, nullptr, 80, 80, nullptr, 12, 1, 32,
                                        8, 96, 64, 1024, 0.088f, KVS_BF16, 0, nullptr, 0, nullptr,
                                        nullptr);
  require(st == KVS_EUNSUPPORTED, "head_dim 96", st);
  require(paged_decode_attention(nullptr, nullptr, nullptr, nullptr, 80, 80, nullptr, 12, 1, 30, 8,
                                 128, 64, 1024, 0.088f, KVS_BF16, 0, nullptr, 0, nullptr,
                                 nullptr) == KVS_EINVAL,
          "heads not a multiple");
  require(paged_decode_attention(nullptr, nullptr, nullptr, nullptr, 80, 80, nullptr, 12, 1, 32, 8,
                                 128, 64, 1024, 0.088f, KVS_BF16, 0, nullptr, 0, nullptr,
                                 nullptr) == KVS_EINVAL,
          "null buffers");
  require(paged_decode_attention(nullptr, nullptr, nullptr, nullptr, 80, 80, nullptr, 8193, 1, 32, 8,
                                 128, 64, 1024, 0.088f, KVS_BF16, 0, nullptr, 0, nullptr,
                                 nullptr) == KVS_EUNSUPPORTED,
          "batch above the largest the decode kernels take");
  require(paged_decode_attention(nullptr, nullptr, nullptr, nullptr, 80, 81, nullptr, 12, 1, 32, 8,
                                 128, 64, 1024, 0.088f, KVS_BF16, 0, nullptr, 0, nullptr,
                                 nullptr) == KVS_EINVAL,
          "walk beyond the table");
  // Misaligned pointers (fake addresses, never dereferenced): rejected
  // before any device work, whatever else the call holds.
  const auto at = [](uintptr_t a) { return reinterpret_cast<void*>(a); };
  int32_t* const i16 = static_cast<int32_t*>(at(0x100000));
  int64_t* const l16 = static_cast<int64_t*>(at(0x100000));
  float* const f16 = static_cast<float*>(at(0x100000));
  require(kv_slot_mapping(i16, static_cast<int64_t*>(at(0x100004)), 8, 8, i16, 4, 4, 16, l16,
                          nullptr) == KVS_EINVAL,
          "positions not 8-byte aligned");
  require(kv_slot_mapping(static_cast<int32_t*>(at(0x100002)), l16, 8, 8, i16, 4, 4, 16, l16,
                          nullptr) == KVS_EINVAL,
          "request indices not 4-byte aligned");
  require(kv_slot_mapping_dcp(i16, l16, 8, 8, i16, 4, 4, 16, 2, 0, 1,
                              static_cast<int64_t*>(at(0x100004)), nullptr) == KVS_EINVAL,
          "dcp slots not 8-byte aligned");
  require(kv_cache_write(at(0x100008), at(0x100000), l16, 8, at(0x100000), at(0x100000), 4, 16,
                         8, 128, KVS_BF16, nullptr) == KVS_EINVAL,
          "new K rows not 16-byte aligned");
  require(kv_cache_write(at(0x100000), at(0x100000), l16, 8, at(0x100000), at(0x100008), 4, 16,
                         8, 128, KVS_BF16, nullptr) == KVS_EINVAL,
          "V cache not 16-byte aligned");
  require(kv_slot_mapping_cache_write(i16, l16, 8, 8, i16, 4, 4, 16, l16, at(0x100000),
                                      at(0x100000), at(0x100004), at(0x100000), 4, 8, 128,
                                      KVS_BF16, nullptr) == KVS_EINVAL,
          "fused write: K cache not 16-byte aligned");
  require(paged_decode_attention(at(0x100008), at(0x100000), at(0x100000), i16, 80, 80, i16, 12, 1,
                                 32, 8, 128, 64, 1024, 0.088f, KVS_BF16, 0, at(0x100000),
                                 SIZE_MAX, f16, nullptr) == KVS_EINVAL,
          "q not 16-byte aligned");
  require(paged_decode_attention(at(0x100000), at(0x100000), at(0x100000), i16, 80, 80, i16, 12, 1,
                                 32, 8, 128, 64, 1024, 0.088f, KVS_BF16, 0, at(0x100008),
                                 SIZE_MAX, f16, nullptr) == KVS_EINVAL,
          "workspace not 16-byte aligned");
  require(paged_decode_attention(at(0x100000), at(0x100000), at(0x100000), i16, 80, 80,
                                 static_cast<int32_t*>(at(0x100002)), 12, 1, 32, 8, 128, 64, 1024,
                                 0.088f, KVS_BF16, 0, at(0x100000), SIZE_MAX, f16,
                                 nullptr) == KVS_EINVAL,
          "seq_lens not 4-byte aligned");
  require(paged_decode_attention_dcp(at(0x100000), at(0x100000), at(0x100000), i16, 80, 80, i16,
                                     12, 1, 32, 8, 128, 64, 1024, 0.088f, KVS_BF16, 2, 0, 1,
                                     at(0x100000), SIZE_MAX, f16,
                                     static_cast<float*>(at(0x100002)), nullptr) == KVS_EINVAL,
          "lse not 4-byte aligned");
  require(paged_decode_attention_append(i16, l16, 8, 8, l16, at(0x100008), at(0x100000),
                                        at(0x100000), at(0x100000), at(0x100000), i16, 80, 80,
                                        i16, 12, 1, 32, 8, 128, 64, 1024, 0.088f, KVS_BF16, 0,
                                        at(0x100000), SIZE_MAX, f16, nullptr) == KVS_EINVAL,
          "append: new K rows not 16-byte aligned");
  require(paged_decode_attention_append(i16, l16, 8, 8, nullptr, at(0x100000), at(0x100000),
                                        at(0x100000), at(0x100000), at(0x100000), i16, 80, 80,
                                        i16, 12, 1, 32, 8, 128, 64, 1024, 0.088f, KVS_BF16, 0,
                                        at(0x100000), SIZE_MAX, f16, nullptr) == KVS_EINVAL,
          "append: no slot buffer");
  require(paged_decode_attention_append(i16, l16, 9, 8, l16, at(0x100000), at(0x100000),
                                        at(0x100000), at(0x100000), at(0x100000), i16, 80, 80,
                                        i16, 12, 1, 32, 8, 128, 64, 1024, 0.088f, KVS_BF16, 0,
                                        at(0x100000), SIZE_MAX, f16, nullptr) == KVS_EINVAL,
          "append: more tokens than slots");
  require(paged_decode_attention_append(nullptr, nullptr, 0, 0, nullptr, nullptr, nullptr,
                                        nullptr, nullptr, nullptr, nullptr, 80, 80, nullptr, 12,
                                        1, 32, 8, 96, 64, 1024, 0.088f, KVS_BF16, 0, nullptr, 0,
                                        nullptr, nullptr) == KVS_EUNSUPPORTED,
          "append: head_dim 96");
  // the entry point without a workspace: argument errors come back before
  // the library looks up its own array (no device needed here)
  require(paged_decode_attention_noalloc(at(0x100008), at(0x100000), at(0x100000), i16, 80, 80,
                                         i16, 12, 1, 32, 8, 128, 64, 1024, 0.088f, KVS_BF16, 0,
                                         f16, nullptr) == KVS_EINVAL,
          "noalloc: q not 16-byte aligned");
  require(paged_decode_attention_noalloc(nullptr, nullptr, nullptr, nullptr, 80, 80, nullptr, 12,
                                         1, 32, 8, 96, 64, 1024, 0.088f, KVS_BF16, 0, nullptr,
                                         nullptr) == KVS_EUNSUPPORTED,
          "noalloc: head_dim 96");
  require(paged_decode_attention_noalloc(at(0x100000), at(0x100000), at(0x100000), i16, 80, 80,
                                         i16, 12, 1, 32, 8, 128, 64, 1024, 0.088f, KVS_BF16, 0,
                                         nullptr, nullptr) == KVS_EINVAL,
          "noalloc: no output");
  require(paged_decode_attention_noalloc(nullptr, nullptr, nullptr, nullptr, 80, 80, nullptr, 0,
                                         1, 32, 8, 128, 64, 1024, 0.088f, KVS_BF16, 0, nullptr,
                                         nullptr) == KVS_OK,
          "noalloc: empty batch");
  require(decode_lse_merge(static_cast<float*>(at(0x100008)), f16, 2, 16, 128, f16, f16,
                           nullptr) == KVS_EINVAL,
          "merge inputs not 16-byte aligned");
  // workspace size query: extreme sizes neither overflow nor trap
  const int32_t big[] = {0, 1, 8192, INT32_MAX};
  for (int32_t B : big)
    for (int32_t Sq : {1, 16, INT32_MAX})
      for (int32_t Hq : {1, 64, INT32_MAX})
        for (int32_t Hkv : {1, 8, INT32_MAX}) {
          const size_t n = paged_decode_attention_workspace_bytes(B, Sq, Hq, Hkv, 128);
          require(B > 0 || n > 0, "workspace for an empty batch", (long)n);
        }
  require(paged_decode_attention_workspace_bytes(-1, 1, 32, 8, 128) == 0, "negative batch");
}

}  // namespace

int main() {
  std::mt19937 rng(20261202);
  check_select_ctx_bucket();
  check_select_batch_bucket(rng);
  check_map_to_kernel_blocks(rng);
  check_swa_tail_trim(rng);
  check_gpu_entry_argument_checks();
  std::printf("ok %d checks\n", g_checks);
  return 0;
}
