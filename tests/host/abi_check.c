/*
 * Host-side check of the C ABI's argument validation, built with the
 * address and undefined-behaviour sanitizers on the host code (see
 * tests/test_host_sanitizers.py). Every call below must be rejected before
 * anything is enqueued, so no GPU is needed and no device memory is touched:
 * the pointers are fake, aligned, non-null addresses that are never
 * dereferenced on the host. Prints one line per check and exits non-zero on
 * the first wrong status.
 */
#include <stdio.h>
#include <stdint.h>
#include <string.h>

#include "hq.h"

#define FAKE ((void *)(uintptr_t)0x100000)
#define FAKE_OFF(n) ((void *)((uintptr_t)0x100000 + (n)))

static int n_checks = 0;

static int expect(const char *what, hq_status got, hq_status want) {
  ++n_checks;
  const char *msg = hq_last_error();
  if (got != want) {
    printf("FAIL %s: status %d, want %d (%s)\n", what, (int)got, (int)want, msg ? msg : "");
    return 1;
  }
  if (want != HQ_OK && (!msg || !msg[0])) {
    printf("FAIL %s: no error message\n", what);
    return 1;
  }
  printf("ok   %s: %s\n", what, want == HQ_OK ? "ok" : msg);
  return 0;
}

static hq_hybrid_kv make_kv(void) {
  hq_hybrid_kv kv;
  memset(&kv, 0, sizeof kv);
  kv.B = 1; kv.Hkv = 2; kv.D = 128; kv.group = 32;
  kv.T = 1000; kv.W = 128; kv.k = 40; kv.t_cap = 896;
  kv.k_codes = FAKE; kv.v_codes = FAKE;
  kv.k_sz = FAKE; kv.v_sz = FAKE; kv.vl_bits = FAKE;
  kv.vl_k = FAKE; kv.vl_v = FAKE; kv.win_k = FAKE; kv.win_v = FAKE;
  kv.hp_dtype = HQ_BF16;
  return kv;
}

int main(void) {
  int bad = 0;
  hq_hybrid_kv kv = make_kv();
  size_t big = (size_t)1 << 40;

  bad |= expect("abi version", hq_abi_version() == HQ_ABI_VERSION ? HQ_OK : HQ_ERR_INVALID_ARG, HQ_OK);
  for (int s = -1; s <= 5; ++s) {
    const char *t = hq_status_string((hq_status)s);
    bad |= expect("status string", (t && t[0]) ? HQ_OK : HQ_ERR_INVALID_ARG, HQ_OK);
  }

  /* decode */
  bad |= expect("decode null kv", hq_decode_attn(FAKE, HQ_BF16, 8, NULL, 0.f, 0, FAKE, NULL, FAKE, big, NULL),
                HQ_ERR_INVALID_ARG);
  kv.D = 96;
  bad |= expect("decode D", hq_decode_attn(FAKE, HQ_BF16, 8, &kv, 0.f, 0, FAKE, NULL, FAKE, big, NULL),
                HQ_ERR_UNSUPPORTED);
  kv = make_kv(); kv.k = 900;
  bad |= expect("decode k > T - W", hq_decode_attn(FAKE, HQ_BF16, 8, &kv, 0.f, 0, FAKE, NULL, FAKE, big, NULL),
                HQ_ERR_INVALID_ARG);
  kv = make_kv(); kv.t_cap = 880;
  bad |= expect("decode t_cap", hq_decode_attn(FAKE, HQ_BF16, 8, &kv, 0.f, 0, FAKE, NULL, FAKE, big, NULL),
                HQ_ERR_INVALID_ARG);
  kv = make_kv(); kv.v_sz = FAKE_OFF(2);
  bad |= expect("decode v_sz alignment", hq_decode_attn(FAKE, HQ_BF16, 8, &kv, 0.f, 0, FAKE, NULL, FAKE, big, NULL),
                HQ_ERR_INVALID_ARG);
  kv = make_kv(); kv.flags = HQ_KV_DROP_INT4; kv.T = 800; kv.W = 0; kv.k = 0;
  bad |= expect("decode empty softmax", hq_decode_attn(FAKE, HQ_BF16, 8, &kv, 0.f, 0, FAKE, NULL, FAKE, big, NULL),
                HQ_ERR_INVALID_ARG);
  kv = make_kv();
  bad |= expect("decode Hq % Hkv", hq_decode_attn(FAKE, HQ_BF16, 7, &kv, 0.f, 0, FAKE, NULL, FAKE, big, NULL),
                HQ_ERR_INVALID_ARG);
  bad |= expect("decode workspace", hq_decode_attn(FAKE, HQ_BF16, 8, &kv, 0.f, 0, FAKE, NULL, FAKE, 8, NULL),
                HQ_ERR_WORKSPACE);
  bad |= expect("decode splits", hq_decode_attn(FAKE, HQ_BF16, 8, &kv, 0.f, -3, FAKE, NULL, FAKE, big, NULL),
                HQ_ERR_INVALID_ARG);
  bad |= expect("decode workspace size", hq_decode_workspace_size(&kv, 8, 0) > 0 ? HQ_OK : HQ_ERR_INVALID_ARG,
                HQ_OK);
  bad |= expect("decode step R", hq_decode_step(FAKE, HQ_BF16, 8, &kv, 0.f, 0, FAKE, NULL, FAKE, big, FAKE, 0, 0,
                                               1, NULL), HQ_ERR_INVALID_ARG);
  bad |= expect("decode step step < 0", hq_decode_step(FAKE, HQ_BF16, 8, &kv, 0.f, 0, FAKE, NULL, FAKE, big, FAKE,
                                                      64, -1, 1, NULL), HQ_ERR_INVALID_ARG);

  /* quantize, gather, bitmap */
  bad |= expect("quantize group", hq_quantize_kv(FAKE, HQ_BF16, 2, 10, 128, 16, 2560, 128, FAKE, FAKE,
                                                HQ_LAYOUT_ROWS, 64, 0, NULL), HQ_ERR_UNSUPPORTED);
  bad |= expect("quantize rows", hq_quantize_kv(FAKE, HQ_BF16, 2, 10, 128, 32, 2560, 128, FAKE, FAKE,
                                               HQ_LAYOUT_ROWS, 64, 60, NULL), HQ_ERR_INVALID_ARG);
  bad |= expect("quantize dtype", hq_quantize_kv(FAKE, (hq_dtype)9, 2, 10, 128, 32, 2560, 128, FAKE, FAKE,
                                                HQ_LAYOUT_ROWS, 64, 0, NULL), HQ_ERR_INVALID_ARG);
  bad |= expect("quantize dtype < 0", hq_quantize_kv(FAKE, (hq_dtype)-1, 2, 10, 128, 32, 2560, 128, FAKE, FAKE,
                                                    HQ_LAYOUT_ROWS, 64, 0, NULL), HQ_ERR_INVALID_ARG);
  bad |= expect("quantize layout", hq_quantize_kv(FAKE, HQ_BF16, 2, 10, 128, 32, 2560, 128, FAKE, FAKE,
                                                 (hq_code_layout)5, 64, 0, NULL), HQ_ERR_INVALID_ARG);
  bad |= expect("quantize empty", hq_quantize_kv(FAKE, HQ_BF16, 2, 0, 128, 32, 2560, 128, FAKE, FAKE,
                                                HQ_LAYOUT_ROWS, 64, 0, NULL), HQ_OK);
  bad |= expect("quantize pair tile rows", hq_quantize_kv_pair(FAKE, FAKE, HQ_BF16, 2, 10, 128, 32, 1280, 128,
                                                              FAKE, FAKE, FAKE, FAKE, 72, 0, NULL),
                HQ_ERR_INVALID_ARG);
  bad |= expect("gather null idx", hq_gather_rows(FAKE, HQ_BF16, 2, 100, 128, NULL, 5, FAKE, NULL),
                HQ_ERR_INVALID_ARG);
  bad |= expect("bitmap t_cap", hq_vl_bitmap(FAKE, 2, 5, 100, FAKE, NULL), HQ_ERR_INVALID_ARG);

  /* detectors */
  int ran = 7;
  bad |= expect("detect R", hq_detect_vlines(NULL, FAKE, HQ_BF16, 1, 32, 2, 128, 0, 0, 0, FAKE, 1000, 900, 45,
                                            HQ_DETECT_MATMUL, FAKE, NULL, &ran, FAKE, big, NULL),
                HQ_ERR_INVALID_ARG);
  bad |= expect("detect method", hq_detect_vlines(NULL, FAKE, HQ_BF16, 1, 32, 2, 128, 64, 63, 0, FAKE, 1000, 900,
                                                 45, (hq_detect_method)3, FAKE, NULL, &ran, FAKE, big, NULL),
                HQ_ERR_INVALID_ARG);
  kv = make_kv();
  bad |= expect("decode q dtype", hq_decode_attn(FAKE, (hq_dtype)-7, 8, &kv, 0.f, 0, FAKE, NULL, FAKE, big, NULL),
                HQ_ERR_INVALID_ARG);
  bad |= expect("detect nothing to do", hq_detect_vlines(NULL, FAKE, HQ_BF16, 1, 32, 2, 128, 64, 5, 0, FAKE, 1000,
                                                        900, 45, HQ_DETECT_MATMUL, FAKE, NULL, &ran, FAKE, big,
                                                        NULL), HQ_OK);
  bad |= expect("detect ran flag", ran == 0 ? HQ_OK : HQ_ERR_INVALID_ARG, HQ_OK);
  bad |= expect("detect cache k_top", hq_detect_vlines_cache(NULL, FAKE, HQ_BF16, 8, 64, 63, 0, &kv, 800, 801,
                                                            FAKE, NULL, &ran, FAKE, big, NULL),
                HQ_ERR_INVALID_ARG);
  bad |= expect("detect mass dtype", hq_detect_vlines_mass(NULL, FAKE, HQ_F32, 1, 32, 2, 128, 64, 63, 0, FAKE,
                                                          1000, 900, 45, 0.f, FAKE, NULL, &ran, FAKE, big, NULL),
                HQ_ERR_UNSUPPORTED);

  /* prefill */
  bad |= expect("prefill D", hq_prefill_attn(FAKE, FAKE, FAKE, HQ_BF16, 1, 8, 2, 1000, 64, 32, 128, FAKE, 50, 0.f,
                                            FAKE, NULL, FAKE, big, NULL), HQ_ERR_UNSUPPORTED);
  bad |= expect("prefill k", hq_prefill_attn(FAKE, FAKE, FAKE, HQ_BF16, 1, 8, 2, 1000, 128, 32, 128, FAKE, 1001,
                                            0.f, FAKE, NULL, FAKE, big, NULL), HQ_ERR_INVALID_ARG);
  bad |= expect("prefill workspace", hq_prefill_attn(FAKE, FAKE, FAKE, HQ_BF16, 1, 8, 2, 1000, 128, 32, 128, FAKE,
                                                    50, 0.f, FAKE, NULL, FAKE, 64, NULL), HQ_ERR_WORKSPACE);

  bad |= expect("prefill i8 D", hq_prefill_attn_i8(FAKE, FAKE, FAKE, HQ_BF16, 1, 8, 2, 1000, 64, 32, 128, FAKE, 50,
                                                  0.f, FAKE, NULL, FAKE, big, NULL), HQ_ERR_UNSUPPORTED);
  bad |= expect("prefill i8 T", hq_prefill_attn_i8(FAKE, FAKE, FAKE, HQ_BF16, 1, 2, 2, (int64_t)1 << 23, 128, 32, 128,
                                                  NULL, 0, 0.f, FAKE, NULL, FAKE, big, NULL), HQ_ERR_UNSUPPORTED);
  bad |= expect("prefill i8 workspace", hq_prefill_attn_i8(FAKE, FAKE, FAKE, HQ_BF16, 1, 8, 2, 1000, 128, 32, 128,
                                                          FAKE, 50, 0.f, FAKE, NULL, FAKE, 64, NULL),
                HQ_ERR_WORKSPACE);

  /* rolling-cache VL update (T - W = 872 positions, ring of W rows) */
  bad |= expect("vl update null kv", hq_vl_update(NULL, FAKE, 800, FAKE, 872, NULL), HQ_ERR_INVALID_ARG);
  bad |= expect("vl update p0 past T - W", hq_vl_update(&kv, FAKE, 873, FAKE, 872, NULL), HQ_ERR_INVALID_ARG);
  bad |= expect("vl update p0 before the ring", hq_vl_update(&kv, FAKE, 700, FAKE, 872, NULL), HQ_ERR_INVALID_ARG);
  bad |= expect("vl update stride", hq_vl_update(&kv, FAKE, 872, FAKE, 871, NULL), HQ_ERR_INVALID_ARG);
  bad |= expect("vl update no-op", hq_vl_update(&kv, FAKE, 872, FAKE, 872, NULL), HQ_OK);

  bad |= expect("vl redetect null kv", hq_vl_redetect(NULL, FAKE, 800, FAKE, HQ_BF16, 8, 64, FAKE, big, NULL), HQ_ERR_INVALID_ARG);
  bad |= expect("vl redetect p0 past T - W", hq_vl_redetect(&kv, FAKE, 873, FAKE, HQ_BF16, 8, 64, FAKE, big, NULL),
                HQ_ERR_INVALID_ARG);
  bad |= expect("vl redetect R", hq_vl_redetect(&kv, FAKE, 872, FAKE, HQ_BF16, 8, 0, FAKE, big, NULL), HQ_ERR_INVALID_ARG);
  bad |= expect("vl redetect dtype", hq_vl_redetect(&kv, FAKE, 872, FAKE, HQ_F16, 8, 64, FAKE, big, NULL), HQ_ERR_INVALID_ARG);
  bad |= expect("vl redetect workspace size", hq_vl_redetect_workspace_size(&kv) == 2 * (40 + 1024) * 8 ? HQ_OK
                                                                                                  : HQ_ERR_INVALID_ARG,
                HQ_OK);
  bad |= expect("vl redetect no-op", hq_vl_redetect(&kv, FAKE, 872, FAKE, HQ_BF16, 8, 64, FAKE, big, NULL), HQ_OK);

  /* allocation-free decode: rejected before any device is touched */
  bad |= expect("noalloc null kv", hq_decode_attn_noalloc(FAKE, HQ_BF16, 8, NULL, 0.f, 0, FAKE, NULL, NULL),
                HQ_ERR_INVALID_ARG);
  bad |= expect("noalloc Hq", hq_decode_attn_noalloc(FAKE, HQ_BF16, 7, &kv, 0.f, 0, FAKE, NULL, NULL),
                HQ_ERR_INVALID_ARG);

  /* stream read */
  bad |= expect("stream read size", hq_stream_read(FAKE, 4100, FAKE, NULL), HQ_ERR_INVALID_ARG);
  bad |= expect("stream read empty", hq_stream_read(FAKE, 0, FAKE, NULL), HQ_OK);

  printf("%d checks, %s\n", n_checks, bad ? "FAILED" : "ALL_OK");
  return bad ? 1 : 0;
}
