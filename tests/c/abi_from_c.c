/* The C ABI used from a plain C99 program (built with gcc, no HIP compiler,
 * no Python): version, status strings, workspace sizing and the host-side
 * rejections of mla_decode_plan and mla_decode_run_noalloc, none of which
 * needs a device.  Prints one line per check; exit status 0 when all pass. */
#include <stdio.h>
#include <string.h>

#include "mla_decode.h"

static int failures = 0;

/* The README's usage example, compiled here so that it keeps to the header;
 * not called (it needs a device). */
mla_status example_step(const void* q, const void* kv, const int32_t* qo_indptr, const int32_t* kv_indptr,
                        const int32_t* kv_indices, const float* kv_scale, void* out, hipStream_t stream);
mla_status example_step(const void* q, const void* kv, const int32_t* qo_indptr, const int32_t* kv_indptr,
                        const int32_t* kv_indices, const float* kv_scale, void* out, hipStream_t stream) {
  mla_decode_params p = {0};
  p.batch = 64; p.total_q = 64;
  p.num_heads = 16; p.num_kv_heads = 1; p.qk_dim = 576; p.v_dim = 512; p.page_size = 1;
  p.q_dtype = MLA_DTYPE_BF16; p.kv_dtype = MLA_DTYPE_FP8_E4M3FN;
  size_t bytes = mla_decode_workspace_size(&p);
  void* ws;
  if (hipMalloc(&ws, bytes) != hipSuccess) return MLA_ERR_HIP;
  mla_decode_plan_t plan;
  mla_status st = mla_decode_plan(&p, ws, bytes, stream, &plan);
  if (st != MLA_OK) return st;
  st = mla_decode_run(&plan, q, kv, qo_indptr, kv_indptr, kv_indices, NULL, kv_scale, 1.0f / 24.0f, out, stream);
  if (st != MLA_OK) fprintf(stderr, "%s\n", mla_status_string(st));
  return st;
}

static void check(int ok, const char* what) {
  printf("%s %s\n", ok ? "ok  " : "FAIL", what);
  if (!ok) ++failures;
}

static mla_decode_params base_params(void) {
  mla_decode_params p;
  memset(&p, 0, sizeof p);
  p.batch = 64;
  p.total_q = 64;
  p.num_heads = 16;
  p.num_kv_heads = 1;
  p.qk_dim = 576;
  p.v_dim = 512;
  p.page_size = 1;
  p.q_dtype = MLA_DTYPE_BF16;
  p.kv_dtype = MLA_DTYPE_FP8_E4M3FN;
  p.num_units = 256;
  return p;
}

int main(void) {
  check(mla_decode_abi_version() == MLA_DECODE_ABI_VERSION, "abi version matches the header");
  check(strncmp(mla_status_string(MLA_ERR_WORKSPACE), "MLA_ERR_WORKSPACE", 17) == 0, "status string");

  mla_decode_params p = base_params();
  /* counters (64 + 8 int32, padded to 256 B) and 2 * 256 share slots plus 4 per sequence of
     float32 O [16, 512] and lse [16] */
  const size_t slots = 2 * 256 + 64 * 4;
  const size_t expect = 512 + slots * 16 * 512 * 4 + slots * 16 * 4;
  check(mla_decode_workspace_size(&p) == expect, "workspace size of 64 sequences over 256 shares");

  mla_decode_plan_t plan;
  p.num_heads = 8;
  check(mla_decode_workspace_size(&p) == 0, "8 heads: no workspace size");
  check(mla_decode_plan(&p, (void*)4096, (size_t)1 << 30, NULL, &plan) == MLA_ERR_UNSUPPORTED,
        "8 heads: plan is MLA_ERR_UNSUPPORTED");
  p = base_params();
  p.q_dtype = MLA_DTYPE_FP8_E4M3FN;
  p.kv_dtype = MLA_DTYPE_BF16;
  check(mla_decode_plan(&p, (void*)4096, (size_t)1 << 30, NULL, &plan) == MLA_ERR_UNSUPPORTED,
        "fp8 Q over bf16 KV: MLA_ERR_UNSUPPORTED");
  p = base_params();
  check(mla_decode_plan(&p, (void*)4100, (size_t)1 << 30, NULL, &plan) == MLA_ERR_WORKSPACE,
        "misaligned workspace: MLA_ERR_WORKSPACE");
  check(mla_decode_plan(&p, (void*)4096, 4096, NULL, &plan) == MLA_ERR_WORKSPACE,
        "short workspace: MLA_ERR_WORKSPACE");
  check(mla_decode_plan(NULL, (void*)4096, (size_t)1 << 30, NULL, &plan) == MLA_ERR_INVALID_ARG,
        "no params: MLA_ERR_INVALID_ARG");
  p.num_units = 4096; /* 2 * 4096 share slots: beyond the no-alloc array */
  check(mla_decode_run_noalloc(&p, (void*)4096, (void*)4096, (const int32_t*)4096, (const int32_t*)4096,
                               (const int32_t*)4096, NULL, NULL, (const float*)4096, 1.0f / 24.0f,
                               (void*)4096, NULL, NULL) == MLA_ERR_WORKSPACE,
        "no-alloc beyond its array: MLA_ERR_WORKSPACE");
  return failures == 0 ? 0 : 1;
}
