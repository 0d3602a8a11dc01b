// Host-only exercise of libwandit's argument validation, built with
// AddressSanitizer on the host side (tests/test_asan_host.py).  Every call
// below fails validation or touches host memory only, so no GPU is needed:
// the sanitizer checks the host code's reads and writes (the I2V mask helper
// filling a caller buffer, the walk over the host array of block descriptors,
// the status strings, the size functions).
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "wan_dit.h"

static int fails = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++fails;                                                         \
    }                                                                  \
  } while (0)

static wan_cfg_t cfg(int dim, int heads, int ffn, int n_blocks, int in_ch, int img_len, int dtype) {
  wan_cfg_t c;
  memset(&c, 0, sizeof(c));
  c.dim = dim; c.heads = heads; c.head_dim = dim / heads; c.ffn = ffn; c.n_blocks = n_blocks;
  c.in_ch = in_ch; c.out_ch = 16; c.freq_dim = 256; c.text_len = 512; c.img_len = img_len;
  c.img_feat = 1280; c.eps = 1e-6f; c.dtype = dtype; c.attn8 = 0;
  return c;
}

int main() {
  // status strings (static storage)
  for (int st = -7; st <= 1; ++st) EXPECT(strlen(wan_status_str(st)) > 0);

  // the five workloads' sizes, and invalid shapes
  wan_cfg_t c13 = cfg(1536, 12, 8960, 30, 16, 0, WAN_BF16);
  wan_cfg_t c14 = cfg(5120, 40, 13824, 40, 36, 257, WAN_BF16);
  wan_cfg_t ctiny = cfg(128, 2, 512, 1, 16, 0, WAN_F32);
  ctiny.text_len = 32;
  EXPECT(wan_workspace_bytes(&c13, 2, 21, 60, 104) > 0);
  EXPECT(wan_workspace_bytes(&c14, 1, 21, 90, 160) > 0);
  EXPECT(wan_workspace_bytes(&ctiny, 1, 2, 16, 16) > 0);
  EXPECT(wan_workspace_bytes(&c13, 1, 21, 59, 104) == 0);      // odd H/8
  EXPECT(wan_workspace_bytes(&c13, 9, 21, 60, 104) == 0);      // B > 8
  EXPECT(wan_workspace_bytes(nullptr, 1, 21, 60, 104) == 0);
  EXPECT(wan_kv_cache_bytes(&c14, 1) > 0 && wan_kv_cache_bytes(&c14, 0) == 0);
  EXPECT(wan_sample_workspace_bytes(&c13, 2, 21, 60, 104) > wan_workspace_bytes(&c13, 2, 21, 60, 104));
  EXPECT(wan_block_fp8_bytes(&c13) > 0 && wan_block_fp8_bytes(&ctiny) == 0);
  EXPECT(wan_model_fp8_bytes(&c14) == 40 * wan_block_fp8_bytes(&c14));
  EXPECT(wan_attention_8bit_workspace_bytes(1, 12, 32760, 32760) > 0);
  EXPECT(wan_dit_block_noalloc_bytes(&c13, 1, 2, 30, 52) > 0);
  EXPECT(wan_dit_block_noalloc_bytes(&c13, 1, 21, 30, 52) > WAN_NOALLOC_SCRATCH_BYTES);

  // the I2V mask helper writes exactly 4 * lat_f * H8 * W8 floats of a host buffer
  const int lat_f = 21, H8 = 6, W8 = 4, frames = 81;
  uint8_t *fm = (uint8_t *)malloc(frames);
  memset(fm, 0, frames);
  fm[0] = 1;
  float *mask = (float *)malloc(sizeof(float) * 4 * lat_f * H8 * W8);
  EXPECT(wan_i2v_mask(fm, frames, lat_f, H8, W8, mask) == WAN_OK);
  int ones = 0;
  for (int i = 0; i < 4 * lat_f * H8 * W8; ++i) ones += mask[i] == 1.0f;
  EXPECT(ones == 4 * H8 * W8);                                   // frame 0 only, all 4 channels
  EXPECT(wan_i2v_mask(fm, 80, lat_f, H8, W8, mask) == WAN_ERR_SHAPE);
  EXPECT(wan_i2v_mask(nullptr, frames, lat_f, H8, W8, mask) == WAN_ERR_NULL);
  free(mask);
  free(fm);

  // the step walks the host array of n_blocks block descriptors: a NULL
  // weight in the last one must be found (and nothing read past the array)
  void *dummy = (void *)256;   // never dereferenced: every call below fails validation first
  wan_cfg_t c3 = cfg(256, 2, 512, 3, 16, 0, WAN_BF16);
  c3.text_len = 40;
  wan_block_weights_t *blocks = (wan_block_weights_t *)malloc(sizeof(wan_block_weights_t) * 3);
  for (int i = 0; i < 3; ++i) {
    const void **p = (const void **)&blocks[i];
    for (size_t k = 0; k < sizeof(wan_block_weights_t) / sizeof(void *); ++k) p[k] = dummy;
    blocks[i].ca_wkv_img = nullptr;
    blocks[i].ca_bkv_img = nullptr;
  }
  blocks[2].ffn_w2 = nullptr;
  wan_model_weights_t mw;
  memset(&mw, 0, sizeof(mw));
  mw.patch_w = mw.patch_b = mw.head_w = mw.head_b = dummy;
  mw.tmlp.w1 = mw.tmlp.b1 = mw.tmlp.w2 = mw.tmlp.b2 = dummy;
  mw.blocks = blocks;
  EXPECT(wan_dit_step_fwd(&c3, (const float *)dummy, (const float *)dummy, 2, 3, 8, 12, dummy, nullptr,
                          &mw, (float *)dummy, dummy, (size_t)1 << 40, nullptr) == WAN_ERR_NULL);
  blocks[2].ffn_w2 = dummy;
  // I2V inputs inconsistent with the configuration
  EXPECT(wan_dit_step_fwd(&c3, (const float *)dummy, (const float *)dummy, 2, 3, 8, 12, dummy, dummy,
                          &mw, (float *)dummy, dummy, (size_t)1 << 40, nullptr) == WAN_ERR_CONFIG);
  // a workspace one byte short
  const size_t need = wan_workspace_bytes(&c3, 2, 3, 8, 12);
  EXPECT(wan_dit_step_fwd(&c3, (const float *)dummy, (const float *)dummy, 2, 3, 8, 12, dummy, nullptr,
                          &mw, (float *)dummy, dummy, need - 1, nullptr) == WAN_ERR_WORKSPACE);
  // dtype, shape and NULL errors of the other entry points
  wan_cfg_t bad = c3;
  bad.dtype = 7;
  EXPECT(wan_dit_block_fwd(&bad, (float *)dummy, 1, 2, 4, 6, (const float *)dummy, &blocks[0], dummy,
                           nullptr, dummy, (size_t)1 << 40, nullptr) == WAN_ERR_DTYPE);
  bad = c3;
  bad.heads = 3;                                                 // dim != heads * head_dim
  EXPECT(wan_dit_block_fwd(&bad, (float *)dummy, 1, 2, 4, 6, (const float *)dummy, &blocks[0], dummy,
                           nullptr, dummy, (size_t)1 << 40, nullptr) == WAN_ERR_SHAPE);
  EXPECT(wan_dit_block_fwd_noalloc(&c13, (float *)dummy, 1, 21, 30, 52, (const float *)dummy, &blocks[0],
                                   dummy, nullptr, nullptr) == WAN_ERR_WORKSPACE);
  EXPECT(wan_tmlp_fwd(&c3, nullptr, 1, &mw.tmlp, (float *)dummy, dummy, 1 << 20, nullptr) == WAN_ERR_NULL);
  EXPECT(wan_ln_modulate_fwd((const float *)dummy, 1, 4, 8, (const float *)dummy, 5, 1e-6f, dummy,
                             nullptr) == WAN_ERR_CONFIG);
  EXPECT(wan_euler_fwd((float *)dummy, (const float *)dummy, 3, 16, 16, 1, 2, 2, 0.1f, 1, 5.0f,
                       nullptr) == WAN_ERR_SHAPE);
  EXPECT(wan_linear_fwd(dummy, dummy, nullptr, dummy, 4, 4, 100, 0, nullptr) == WAN_ERR_SHAPE);
  EXPECT(wan_attention_fwd(dummy, 100, dummy, 256, dummy, 64, 64, dummy, 256, 1, 2, 4, 4, 0, nullptr) ==
         WAN_ERR_SHAPE);
  free(blocks);
  if (fails) {
    fprintf(stderr, "%d expectation(s) failed\n", fails);
    return 1;
  }
  printf("host validation under AddressSanitizer: OK\n");
  return 0;
}
