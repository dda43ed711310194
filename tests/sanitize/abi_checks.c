/*
 * Host-side checks of the C ABI's argument validation, built with the
 * library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_host_sanitizers.py).  Every call here is rejected (or is an
 * empty no-op) before any device work, so the program runs without a GPU;
 * a memory error or undefined behaviour in the validation code aborts it.
 * Pointers are fake, 256-byte-aligned addresses that are never dereferenced.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "tt.h"

#define FAKE ((void*)(uintptr_t)(1u << 20))
#define FAKE2 ((void*)(uintptr_t)(2u << 20))
#define AT(p, n) ((void*)((char*)(p) + (n)))

static int failures = 0;

static void expect(int got, int want, const char* what, int line) {
  if (got != want) {
    fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", line, what, got, want,
            tt_last_error());
    ++failures;
  } else if (want != TT_OK && tt_last_error()[0] == '\0') {
    fprintf(stderr, "line %d: %s failed without a message\n", line, what);
    ++failures;
  }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

static tt_attn_shape shape(int B, int Hq, int Hkv, int d, int S, int dtype) {
  tt_attn_shape s = {B, Hq, Hkv, d, S, dtype};
  return s;
}

static int attn(tt_attn_shape s, const void* q, const int32_t* cl, int maxl, const float* gate,
                void* ws, size_t ws_bytes) {
  return tt_block_attn(&s, q, FAKE, FAKE, FAKE, FAKE, FAKE, cl, maxl, NULL, NULL, NULL, gate, NULL,
                       FAKE, NULL, ws, ws_bytes, NULL);
}

static void attention(void) {
  const size_t big = (size_t)1 << 30;
  EXPECT(attn(shape(1, 32, 3, 128, 16, 0), FAKE, FAKE, 128, NULL, FAKE, big), TT_ERR_INVALID_ARG);
  EXPECT(attn(shape(1, 32, 2, 96, 16, 0), FAKE, FAKE, 128, NULL, FAKE, big), TT_ERR_UNSUPPORTED);
  EXPECT(attn(shape(1, 32, 2, 128, 0, 0), FAKE, FAKE, 128, NULL, FAKE, big), TT_ERR_INVALID_ARG);
  EXPECT(attn(shape(1, 32, 2, 128, 65, 0), FAKE, FAKE, 128, NULL, FAKE, big), TT_ERR_INVALID_ARG);
  EXPECT(attn(shape(1, 32, 2, 128, 16, 7), FAKE, FAKE, 128, NULL, FAKE, big), TT_ERR_INVALID_ARG);
  EXPECT(attn(shape(-1, 32, 2, 128, 16, 0), FAKE, FAKE, 128, NULL, FAKE, big), TT_ERR_INVALID_ARG);
  EXPECT(attn(shape(1, 0, 2, 128, 16, 0), FAKE, FAKE, 128, NULL, FAKE, big), TT_ERR_INVALID_ARG);
  const tt_attn_shape s = shape(2, 32, 2, 128, 16, 0);
  EXPECT(attn(s, NULL, FAKE, 128, NULL, FAKE, big), TT_ERR_INVALID_ARG);
  EXPECT(attn(s, FAKE, NULL, 128, NULL, FAKE, big), TT_ERR_INVALID_ARG);
  EXPECT(attn(s, AT(FAKE, 2), FAKE, 128, NULL, FAKE, big), TT_ERR_INVALID_ARG);
  EXPECT(attn(s, FAKE, FAKE, 128, AT(FAKE, 4), FAKE, big), TT_ERR_INVALID_ARG);
  EXPECT(attn(s, FAKE, FAKE, -1, NULL, FAKE, big), TT_ERR_INVALID_ARG);
  const size_t need = tt_block_attn_workspace_size(&s, 128);
  if (need == 0) { fprintf(stderr, "workspace size 0\n"); ++failures; }
  EXPECT(attn(s, FAKE, FAKE, 128, NULL, FAKE, need - 1), TT_ERR_WORKSPACE);
  EXPECT(attn(s, FAKE, FAKE, 128, NULL, NULL, big), TT_ERR_WORKSPACE);
  EXPECT(attn(shape(0, 32, 2, 128, 16, 0), FAKE, FAKE, 128, NULL, NULL, 0), TT_OK);
  /* workspace sizes grow with the context hint */
  const tt_attn_shape w8 = shape(8, 32, 2, 128, 16, 0);
  if (!(tt_block_attn_workspace_size(&w8, 1024) <= tt_block_attn_workspace_size(&w8, 32768))) {
    fprintf(stderr, "workspace sizes not monotone\n");
    ++failures;
  }
  /* the allocation-free form: a launch beyond its static scratch */
  const tt_attn_shape huge = shape(2048, 64, 8, 128, 64, 0);
  EXPECT(tt_block_attn_noalloc(&huge, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 16, NULL,
                               NULL, NULL, NULL, NULL, FAKE, NULL, NULL),
         TT_ERR_WORKSPACE);
  EXPECT(tt_block_attn_noalloc(&s, NULL, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 128, NULL, NULL,
                               NULL, NULL, NULL, FAKE, NULL, NULL),
         TT_ERR_INVALID_ARG);
  /* the context tower's form */
  EXPECT(tt_ctx_block_attn(&s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, AT(FAKE, 4), 128, NULL,
                           NULL, FAKE, NULL, FAKE, big, NULL),
         TT_ERR_INVALID_ARG);
  EXPECT(tt_ctx_block_attn(&s, FAKE, FAKE, FAKE, FAKE, AT(FAKE, 8), FAKE, FAKE, FAKE, 128, NULL,
                           NULL, FAKE, NULL, FAKE, big, NULL),
         TT_ERR_INVALID_ARG);
  EXPECT(tt_ctx_block_attn(&s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 128, NULL, NULL,
                           FAKE, NULL, FAKE, need - 1, NULL),
         TT_ERR_WORKSPACE);
  EXPECT(tt_ctx_advance(-1, 16, FAKE, FAKE, FAKE, NULL, NULL, NULL), TT_ERR_INVALID_ARG);
  EXPECT(tt_ctx_advance(2, 65, FAKE, FAKE, FAKE, NULL, NULL, NULL), TT_ERR_INVALID_ARG);
  EXPECT(tt_ctx_advance(2, 16, FAKE, FAKE, AT(FAKE, 2), NULL, NULL, NULL), TT_ERR_INVALID_ARG);
  EXPECT(tt_ctx_advance(0, 16, FAKE, FAKE, FAKE, NULL, NULL, NULL), TT_OK);
}

static int unmask(int B, int S, int V, const void* logits, int dtype, int64_t stride, float gamma,
                  float tau, size_t ws_bytes) {
  return tt_confidence_unmask(B, S, V, logits, dtype, stride, gamma, tau, 3, 0, FAKE, FAKE, NULL,
                              NULL, NULL, NULL, NULL, FAKE, ws_bytes, NULL);
}

static void unmasking(void) {
  const size_t mb = (size_t)1 << 20;
  EXPECT(unmask(1, 0, 1024, FAKE, 0, 1024, 0.8f, 1.f, mb), TT_ERR_INVALID_ARG);
  EXPECT(unmask(1, 65, 1024, FAKE, 0, 1024, 0.8f, 1.f, mb), TT_ERR_INVALID_ARG);
  EXPECT(unmask(1, 16, 0, FAKE, 0, 0, 0.8f, 1.f, mb), TT_ERR_INVALID_ARG);
  EXPECT(unmask(1, 16, 1024, FAKE, 0, 100, 0.8f, 1.f, mb), TT_ERR_INVALID_ARG);
  EXPECT(unmask(1, 16, 1024, FAKE, 0, 1024, 0.8f, 0.f, mb), TT_ERR_INVALID_ARG);
  EXPECT(unmask(1, 16, 1024, FAKE, 0, 1024, 0.8f, -1.f, mb), TT_ERR_INVALID_ARG);
  EXPECT(unmask(1, 16, 1024, FAKE, 0, 1024, 0.8f, INFINITY, mb), TT_ERR_INVALID_ARG);
  EXPECT(unmask(1, 16, 1024, FAKE, 0, 1024, NAN, 1.f, mb), TT_ERR_INVALID_ARG);
  EXPECT(unmask(1, 16, 1024, FAKE, 5, 1024, 0.8f, 1.f, mb), TT_ERR_INVALID_ARG);
  EXPECT(unmask(1, 16, 1024, NULL, 0, 1024, 0.8f, 1.f, mb), TT_ERR_INVALID_ARG);
  EXPECT(unmask(1, 16, 1024, FAKE, 0, 1024, 0.8f, 1.f, 1), TT_ERR_WORKSPACE);
  EXPECT(unmask(0, 16, 1024, FAKE, 0, 1024, 0.8f, 1.f, 0), TT_OK);
  EXPECT(tt_sample_unmask(1, 16, 1024, FAKE, 0, 1024, 0.8f, 0.1f, 7, -1, 3, 0, FAKE, FAKE, NULL,
                          NULL, NULL, NULL, NULL, FAKE, mb, NULL),
         TT_ERR_INVALID_ARG);
  EXPECT(tt_sample_unmask(1, 16, 1024, FAKE, 0, 1024, 0.8f, 0.1f, 7, 0, 3, -2, FAKE, FAKE, NULL,
                          NULL, NULL, NULL, NULL, FAKE, mb, NULL),
         TT_ERR_INVALID_ARG);
  if (tt_unmask_workspace_size(64, 16, 131072) < 64 * 16 * 16) {
    fprintf(stderr, "unmask workspace too small\n");
    ++failures;
  }
  EXPECT(tt_timestep_embed(-1, FAKE, FAKE, NULL), TT_ERR_INVALID_ARG);
  EXPECT(tt_timestep_embed(2, NULL, FAKE, NULL), TT_ERR_INVALID_ARG);
  EXPECT(tt_adaln_single(2, 6, 1, FAKE, FAKE, NULL, NULL, FAKE, NULL), TT_ERR_INVALID_ARG);
  EXPECT(tt_adaln_single(2, 8, 0, FAKE, FAKE, NULL, NULL, FAKE, NULL), TT_ERR_INVALID_ARG);
  EXPECT(tt_workspace_clear(NULL, 16, NULL), TT_ERR_INVALID_ARG);
  EXPECT(tt_workspace_clear(NULL, 0, NULL), TT_OK);
}

static void loops(void) {
  const tt_attn_shape s = shape(2, 4, 1, 64, 16, 1);
  const void* layers[1] = {FAKE};
  const void* null_layers[1] = {NULL};
  tt_step_provider empty;
  memset(&empty, 0, sizeof empty);
  const size_t big = (size_t)1 << 30;
  int32_t taken = -5;
  EXPECT(tt_denoise_block(&s, 1, 17, 0.8f, 1.f, 3, 64, layers, layers, FAKE, FAKE, 8, NULL, NULL,
                          NULL, NULL, FAKE, FAKE, NULL, &taken, FAKE, big, NULL),
         TT_ERR_INVALID_ARG);
  EXPECT(tt_denoise_block(&s, 0, 16, 0.8f, 1.f, 3, 64, layers, layers, FAKE, FAKE, 8, NULL, NULL,
                          NULL, &empty, FAKE, FAKE, NULL, &taken, FAKE, big, NULL),
         TT_ERR_INVALID_ARG);
  EXPECT(tt_denoise_block(&s, 1, 16, 0.8f, 1.f, 3, 64, layers, layers, FAKE, FAKE, 8, NULL, NULL,
                          NULL, &empty, FAKE, FAKE, NULL, &taken, FAKE, big, NULL),
         TT_ERR_INVALID_ARG);
  EXPECT(tt_denoise_block(&s, 1, 16, 0.8f, 1.f, 3, 64, null_layers, layers, FAKE, FAKE, 8, NULL,
                          NULL, NULL, NULL, FAKE, FAKE, NULL, &taken, FAKE, big, NULL),
         TT_ERR_INVALID_ARG);
  if (taken != 0) { fprintf(stderr, "steps_taken not cleared\n"); ++failures; }
  EXPECT(tt_denoise_block_resume(&s, 1, -1, 16, 0.8f, 1.f, 0, 9, 0, 3, 64, layers, layers, FAKE,
                                 FAKE, 8, NULL, NULL, NULL, NULL, FAKE, FAKE, NULL, &taken, FAKE,
                                 big, NULL),
         TT_ERR_INVALID_ARG);
  EXPECT(tt_denoise_block_resume(&s, 1, 4, 13, 0.8f, 1.f, 0, 9, 0, 3, 64, layers, layers, FAKE,
                                 FAKE, 8, NULL, NULL, NULL, NULL, FAKE, FAKE, NULL, &taken, FAKE,
                                 big, NULL),
         TT_ERR_INVALID_ARG);
  EXPECT(tt_denoise_block_resume(&s, 1, 4, 12, 0.8f, 1.f, 1, 9, -1, 3, 64, layers, layers, FAKE,
                                 FAKE, 8, NULL, NULL, NULL, NULL, FAKE, FAKE, NULL, &taken, FAKE,
                                 big, NULL),
         TT_ERR_INVALID_ARG);
  if (tt_denoise_workspace_size(&s, 1, 8, 64) == 0) { fprintf(stderr, "denoise ws 0\n"); ++failures; }

  const tt_attn_shape g = shape(2, 4, 1, 64, 16, 0);
  void* glayers[1] = {FAKE};
  void* null_glayers[1] = {NULL};
  tt_gen_provider gempty;
  memset(&gempty, 0, sizeof gempty);
  EXPECT(tt_generate(&g, 1, 2, 0, 0.8f, 0.1f, 1, 5, 3, 2, 64, glayers, glayers, FAKE, FAKE, FAKE,
                     8, NULL, NULL, NULL, NULL, FAKE, FAKE, NULL, &taken, FAKE, big, NULL),
         TT_ERR_INVALID_ARG);
  EXPECT(tt_generate(&g, 1, -1, 16, 0.8f, 0.1f, 1, 5, 3, 2, 64, glayers, glayers, FAKE, FAKE,
                     FAKE, 8, NULL, NULL, NULL, NULL, FAKE, FAKE, NULL, &taken, FAKE, big, NULL),
         TT_ERR_INVALID_ARG);
  EXPECT(tt_generate(&g, 1, 2, 16, 0.8f, 0.1f, 1, 5, 3, 2, 64, glayers, glayers, FAKE, NULL, FAKE,
                     8, NULL, NULL, NULL, &gempty, FAKE, FAKE, NULL, &taken, FAKE, big, NULL),
         TT_ERR_INVALID_ARG);
  EXPECT(tt_generate(&g, 1, 2, 16, 0.8f, 0.1f, 1, 5, 3, 2, 64, null_glayers, glayers, FAKE, FAKE,
                     FAKE, 8, NULL, NULL, NULL, &gempty, FAKE, FAKE, NULL, &taken, FAKE, big,
                     NULL),
         TT_ERR_INVALID_ARG);
  EXPECT(tt_generate(&g, 1, 2, 16, 0.8f, 0.1f, 1, 5, 3, 2, 64, glayers, glayers, FAKE, FAKE, FAKE,
                     INT32_MAX, NULL, NULL, NULL, &gempty, FAKE, FAKE, NULL, &taken, FAKE, big,
                     NULL),
         TT_ERR_INVALID_ARG);
}

static int mamba(tt_mamba_shape m, const void* xbc, const float* ss, void* cso, size_t ws) {
  return tt_mamba_block_scan(&m, xbc, FAKE, FAKE, ss, FAKE, NULL, FAKE, NULL, NULL, NULL, FAKE,
                             cso, NULL, FAKE, ws, NULL);
}

static void mamba_and_sublayer(void) {
  const size_t big = (size_t)1 << 30;
  const tt_mamba_shape ok_shape = {2, 8, 64, 128, 2, 4, 16, 0};
  tt_mamba_shape m = ok_shape;
  m.n_groups = 3;
  EXPECT(mamba(m, FAKE, FAKE, NULL, big), TT_ERR_INVALID_ARG);
  m = ok_shape; m.head_dim = 48;
  EXPECT(mamba(m, FAKE, FAKE, NULL, big), TT_ERR_UNSUPPORTED);
  m = ok_shape; m.conv_width = 1;
  EXPECT(mamba(m, FAKE, FAKE, NULL, big), TT_ERR_INVALID_ARG);
  m = ok_shape; m.block_size = 65;
  EXPECT(mamba(m, FAKE, FAKE, NULL, big), TT_ERR_INVALID_ARG);
  EXPECT(mamba(ok_shape, NULL, FAKE, NULL, big), TT_ERR_INVALID_ARG);
  EXPECT(mamba(ok_shape, FAKE, AT(FAKE, 8), NULL, big), TT_ERR_INVALID_ARG);
  EXPECT(mamba(ok_shape, FAKE, FAKE, FAKE, big), TT_ERR_INVALID_ARG);
  EXPECT(mamba(ok_shape, FAKE, FAKE, NULL, 16), TT_ERR_WORKSPACE);
  m = ok_shape; m.batch = 0;
  EXPECT(mamba(m, FAKE, FAKE, NULL, big), TT_OK);

  const tt_attn_shape s = shape(2, 4, 2, 64, 16, 0);
  const tt_attn_shape s32 = shape(2, 4, 2, 64, 16, 1);
  EXPECT(tt_ln_modulate(&s32, 256, FAKE, FAKE, FAKE, NULL, FAKE2, NULL), TT_ERR_UNSUPPORTED);
  EXPECT(tt_ln_modulate(&s, 200, FAKE, FAKE, FAKE, NULL, FAKE2, NULL), TT_ERR_UNSUPPORTED);
  EXPECT(tt_ln_modulate(&s, 256, NULL, FAKE, FAKE, NULL, FAKE2, NULL), TT_ERR_INVALID_ARG);
  EXPECT(tt_ln_modulate(&s, 256, FAKE, FAKE, FAKE, NULL, AT(FAKE, 256), NULL), TT_ERR_INVALID_ARG);
  EXPECT(tt_qkv_proj(&s, 256, FAKE, FAKE, NULL, FAKE, AT(FAKE2, 4096), AT(FAKE2, 8192), NULL),
         TT_ERR_INVALID_ARG);
  EXPECT(tt_out_proj(&s, 256, FAKE, FAKE, FAKE, FAKE2, NULL, FAKE, NULL), TT_ERR_INVALID_ARG);
  EXPECT(tt_adaln_attn_sublayer(&s, 256, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                FAKE, 64, NULL, FAKE2, FAKE, 256, NULL),
         TT_ERR_WORKSPACE);
  EXPECT(tt_adaln_attn_sublayer(&s, 256, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                FAKE, -1, NULL, FAKE2, FAKE, big, NULL),
         TT_ERR_INVALID_ARG);
  if (tt_adaln_sublayer_workspace_size(&s32, 256, 64) != 0) {
    fprintf(stderr, "fp32 sublayer workspace should be 0\n");
    ++failures;
  }
}

int main(void) {
  if (tt_abi_version() != TT_ABI_VERSION) {
    fprintf(stderr, "ABI version %d, header %d\n", tt_abi_version(), TT_ABI_VERSION);
    return 1;
  }
  attention();
  unmasking();
  loops();
  mamba_and_sublayer();
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("abi checks ok\n");
  return 0;
}
