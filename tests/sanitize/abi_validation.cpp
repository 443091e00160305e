// Drives the argument checks of the C ABI (the cases of the Python ABI tests
// plus size extremes) in a build whose host code carries AddressSanitizer and
// UndefinedBehaviorSanitizer. Every call must return its status before any
// launch; exit status 0 when every status matches.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "kvq.h"

static int failures = 0;
#define EXPECT(call, want)                                                              \
  do {                                                                                  \
    const int got_ = (int)(call);                                                       \
    if (got_ != (int)(want)) {                                                          \
      fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #call, \
              got_, (int)(want));                                                       \
      ++failures;                                                                       \
    }                                                                                   \
  } while (0)

static kvq_config kivi() {
  kvq_config c;
  memset(&c, 0, sizeof(c));
  c.d_head = 128; c.n_kv_heads = 8; c.n_q_heads = 32; c.k_bits = 4; c.v_bits = 4;
  c.k_axis = KVQ_AXIS_CHANNEL; c.k_group_tokens = 32; c.k_residual_tokens = 32;
  c.v_group_channels = 128;
  return c;
}

static kvq_config token8() {
  kvq_config c = kivi();
  c.k_bits = c.v_bits = 8; c.k_axis = KVQ_AXIS_TOKEN; c.k_group_tokens = 0; c.k_residual_tokens = 0;
  return c;
}

int main() {
  kvq_sizes s;
  // configurations
  kvq_config c = kivi();
  EXPECT(kvq_cache_sizes(&c, 3, 4096, &s), KVQ_OK);
  EXPECT(kvq_cache_sizes(nullptr, 3, 4096, &s), KVQ_EINVAL);
  EXPECT(kvq_cache_sizes(&c, 3, 4096, nullptr), KVQ_EINVAL);
  c = kivi(); c.k_bits = 3; EXPECT(kvq_cache_sizes(&c, 2, 256, &s), KVQ_EUNSUPPORTED);
  c = kivi(); c.d_head = 64; EXPECT(kvq_cache_sizes(&c, 2, 256, &s), KVQ_EUNSUPPORTED);
  c = kivi(); c.n_q_heads = 12; EXPECT(kvq_cache_sizes(&c, 2, 256, &s), KVQ_EINVAL);
  c = kivi(); c.n_kv_heads = 0; EXPECT(kvq_cache_sizes(&c, 2, 256, &s), KVQ_EINVAL);
  c = kivi(); c.n_kv_heads = -8; EXPECT(kvq_cache_sizes(&c, 2, 256, &s), KVQ_EINVAL);
  c = kivi(); c.n_q_heads = 8 * 16; EXPECT(kvq_cache_sizes(&c, 2, 256, &s), KVQ_EUNSUPPORTED);
  c = kivi(); c.k_residual_tokens = 48; EXPECT(kvq_cache_sizes(&c, 2, 256, &s), KVQ_EINVAL);
  c = kivi(); c.k_sparse_per_vector = 3; EXPECT(kvq_cache_sizes(&c, 2, 256, &s), KVQ_EUNSUPPORTED);
  c = kivi(); c.k_axis = 7; EXPECT(kvq_cache_sizes(&c, 2, 256, &s), KVQ_EINVAL);
  c = kivi(); c.k_format = 9; c.v_format = 9; EXPECT(kvq_cache_sizes(&c, 2, 256, &s), KVQ_EINVAL);
  c = token8(); c.k_format = c.v_format = KVQ_FORMAT_FP8; c.k_scale = 1.f; c.v_scale = NAN;
  EXPECT(kvq_cache_sizes(&c, 2, 256, &s), KVQ_EINVAL);
  c.v_scale = 1.f; EXPECT(kvq_cache_sizes(&c, 2, 256, &s), KVQ_OK);
  // shapes and size extremes (64-bit arithmetic throughout)
  c = kivi();
  EXPECT(kvq_cache_sizes(&c, 0, 256, &s), KVQ_EINVAL);
  EXPECT(kvq_cache_sizes(&c, -1, 256, &s), KVQ_EINVAL);
  EXPECT(kvq_cache_sizes(&c, 2, 70, &s), KVQ_EINVAL);
  EXPECT(kvq_cache_sizes(&c, 2, -32, &s), KVQ_EINVAL);
  EXPECT(kvq_cache_sizes(&c, 2, (int64_t)1 << 40, &s), KVQ_EUNSUPPORTED);
  EXPECT(kvq_cache_sizes(&c, 0x7fffffff, 1 << 24, &s), KVQ_EUNSUPPORTED);   // past 2^44 slots
  EXPECT(kvq_cache_sizes(&c, 1 << 17, 1 << 24, &s), KVQ_OK);                  // 2^44 - exactly the bound
  if (s.total_bytes < s.k_codes || s.k_codes != ((uint64_t)1 << 44) * 128 / 2) {
    fprintf(stderr, "sizes at the bound\n");
    ++failures;
  }
  if (kvq_workspace_bytes(&c, 1 << 17, 1 << 24) == 0) { fprintf(stderr, "workspace 0\n"); ++failures; }
  c.n_kv_heads = 1 << 20; c.n_q_heads = 1 << 23;
  EXPECT(kvq_cache_sizes(&c, 0x7fffffff, 1 << 24, &s), KVQ_EUNSUPPORTED);
  if (kvq_workspace_bytes(&c, 0x7fffffff, 1 << 24) != 0) { fprintf(stderr, "workspace past the bound\n"); ++failures; }
  c = kivi();
  if (kvq_workspace_bytes(&c, 0, 256) != 0) { fprintf(stderr, "workspace of a bad shape\n"); ++failures; }

  // appends and attention: every error returns before a launch
  char* fake = (char*)((uintptr_t)1 << 20);
  int32_t lens[2] = {60, 0};
  kvq_cache k;
  memset(&k, 0, sizeof(k));
  k.batch = 2; k.max_tokens = 64;
  k.k_codes = k.k_meta = k.k_resid = k.k_sparse = k.v_codes = k.v_meta = fake;
  k.seq_len = (int32_t*)fake; k.len_host = lens;
  int32_t n[2] = {5, 1};
  c = kivi();
  EXPECT(kvq_append(&c, &k, fake, fake, (int32_t*)fake, n, nullptr), KVQ_ECAPACITY);
  n[0] = -1; EXPECT(kvq_append(&c, &k, fake, fake, (int32_t*)fake, n, nullptr), KVQ_EINVAL);
  n[0] = 1; EXPECT(kvq_append(&c, &k, fake, fake, nullptr, n, nullptr), KVQ_EINVAL);
  EXPECT(kvq_append(&c, &k, fake + 2, fake, (int32_t*)fake, n, nullptr), KVQ_EINVAL);
  n[0] = n[1] = 0; EXPECT(kvq_append(&c, &k, nullptr, nullptr, (int32_t*)fake, n, nullptr), KVQ_OK);
  n[0] = 0x7fffffff; n[1] = 0x7fffffff;
  EXPECT(kvq_append(&c, &k, fake, fake, (int32_t*)fake, n, nullptr), KVQ_ECAPACITY);
  kvq_cache k2 = k; k2.k_resid = nullptr; n[0] = 1; n[1] = 1;
  EXPECT(kvq_append(&c, &k2, fake, fake, (int32_t*)fake, n, nullptr), KVQ_EINVAL);
  k2 = k; k2.max_tokens = 70; EXPECT(kvq_append(&c, &k2, fake, fake, (int32_t*)fake, n, nullptr), KVQ_EINVAL);
  k2 = k; k2.len_host = nullptr; EXPECT(kvq_append(&c, &k2, fake, fake, (int32_t*)fake, n, nullptr), KVQ_EINVAL);
  lens[0] = -5; EXPECT(kvq_append(&c, &k, fake, fake, (int32_t*)fake, n, nullptr), KVQ_EINVAL);
  lens[0] = 60;

  const size_t need = kvq_workspace_bytes(&c, 2, 64);
  EXPECT(kvq_decode_attention(&c, &k, fake, (float*)fake, 0.1f, fake, need - 1, nullptr), KVQ_EWORKSPACE);
  EXPECT(kvq_decode_attention(&c, &k, nullptr, (float*)fake, 0.1f, fake, need, nullptr), KVQ_EINVAL);
  EXPECT(kvq_decode_attention(&c, &k, fake, (float*)(fake + 4), 0.1f, fake, need, nullptr), KVQ_EINVAL);
  EXPECT(kvq_decode_attention(&c, &k, fake, (float*)fake, 0.1f, nullptr, need, nullptr), KVQ_EINVAL);
  lens[1] = 65;
  EXPECT(kvq_decode_attention(&c, &k, fake, (float*)fake, 0.1f, fake, need, nullptr), KVQ_EINVAL);
  EXPECT(kvq_decode_attention_noalloc(&c, &k, fake, (float*)fake, 0.1f, nullptr), KVQ_EINVAL);
  EXPECT(kvq_dequantize(&c, &k, fake, fake, nullptr), KVQ_EINVAL);
  lens[1] = 0;
  EXPECT(kvq_dequantize(&c, &k, nullptr, fake, nullptr), KVQ_EINVAL);
  EXPECT(kvq_decode_attention_noalloc(&c, &k, fake, (float*)(fake + 4), 0.1f, nullptr), KVQ_EINVAL);

  // an fp8 cache needs no metadata pointers; an affine one does
  kvq_config f = token8();
  f.k_format = f.v_format = KVQ_FORMAT_FP8; f.k_scale = f.v_scale = 1.f;
  k2 = k; k2.k_meta = k2.v_meta = nullptr; n[0] = 5; n[1] = 1;
  EXPECT(kvq_append(&f, &k2, fake, fake, (int32_t*)fake, n, nullptr), KVQ_ECAPACITY);
  kvq_config t = token8();
  EXPECT(kvq_append(&t, &k2, fake, fake, (int32_t*)fake, n, nullptr), KVQ_EINVAL);

  for (int st = 0; st <= 6; ++st)
    if (!kvq_status_string((kvq_status)st)[0]) ++failures;
  if (failures) fprintf(stderr, "%d check(s) failed\n", failures);
  else printf("all validation checks passed\n");
  return failures ? 1 : 0;
}
