/*
 * Plain-C driver of the library's C ABI (test infrastructure).
 *
 * Reads a finalize workload from a directory written by the test suite,
 * runs moe_finalize (fp32 and packed weights) and moe_finalize_quant_ue8m0
 * through the C ABI on a HIP stream it creates, then hands the two finalize
 * outputs, as two ranks' outputs, to moe_allreduce_residual_rmsnorm (a host
 * array of device pointers, the shared output as the residual). It writes the
 * outputs back for the test to compare with the CPU oracle, and checks that
 * rejected calls return their documented status before touching the GPU.
 *
 * usage: abi_driver DIR
 *   DIR/meta.txt : "T H K P rsf"
 *   DIR/g2.bin (uint16 P*H) idx.bin (int32 T*K) w.bin (float T*K)
 *   DIR/packed.bin (int32 T*K) shared.bin (uint16 T*H) gamma.bin (uint16 H)
 *   -> DIR/out.bin, out_packed.bin (uint16 T*H), q.bin (uint8 T*H),
 *      s.bin (uint8 T*H/128), err.bin (int32), ro.bin, nm.bin (uint16 T*H)
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "moe_finalize.h"

#define CHECK_HIP(x)                                                        \
  do {                                                                      \
    hipError_t e_ = (x);                                                    \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "HIP error %d at line %d\n", (int)e_, __LINE__);      \
      return 2;                                                             \
    }                                                                       \
  } while (0)

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  void* p = malloc(bytes ? bytes : 1);
  size_t got = fread(p, 1, bytes, f);
  fclose(f);
  if (got != bytes) {
    free(p);
    return NULL;
  }
  return p;
}

static int write_file(const char* dir, const char* name, const void* p, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) return -1;
  size_t put = fwrite(p, 1, bytes, f);
  fclose(f);
  return put == bytes ? 0 : -1;
}

static int expect(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "%s: status %d (%s), expected %d\n", what, got,
            moe_finalize_status_string(got), want);
    return 1;
  }
  return 0;
}

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s DIR\n", argv[0]);
    return 2;
  }
  const char* dir = argv[1];
  if (moe_finalize_abi_version() != MOEF_ABI_VERSION) return 3;

  /* rejected calls: no HIP call is made for them */
  int bad = 0;
  bad |= expect(moe_finalize(NULL, 0, NULL, NULL, NULL, NULL, 1.0f, NULL, -1, 4096, 8, NULL, NULL),
                MOEF_ERR_BAD_SHAPE, "negative T");
  bad |= expect(moe_finalize((const uint16_t*)0x1000, 8, (const int32_t*)0x2000,
                             (const float*)0x3000, (const int32_t*)0x4000, NULL, 1.0f,
                             (uint16_t*)0x5000, 4, 4096, 8, NULL, NULL),
                MOEF_ERR_BAD_FORMAT, "both weight formats");
  bad |= expect(moe_finalize_quant_ue8m0((const uint16_t*)0x1000, 8, (const int32_t*)0x2000,
                                         (const float*)0x3000, NULL, NULL, 1.0f,
                                         (uint8_t*)0x5000, (uint8_t*)0x9000, 4, 4104, 8, NULL,
                                         NULL),
                MOEF_ERR_UNSUPPORTED, "hidden not a multiple of 128");
  if (bad) return 4;

  long long T, H, K, P;
  float rsf;
  {
    char path[4096];
    snprintf(path, sizeof path, "%s/meta.txt", dir);
    FILE* f = fopen(path, "r");
    if (!f || fscanf(f, "%lld %lld %lld %lld %f", &T, &H, &K, &P, &rsf) != 5) return 5;
    fclose(f);
  }
  const size_t row = (size_t)H * 2, slots = (size_t)(T * K);
  void* h_g2 = read_file(dir, "g2.bin", (size_t)P * row);
  void* h_idx = read_file(dir, "idx.bin", slots * 4);
  void* h_w = read_file(dir, "w.bin", slots * 4);
  void* h_pk = read_file(dir, "packed.bin", slots * 4);
  void* h_sh = read_file(dir, "shared.bin", (size_t)T * row);
  void* h_gam = read_file(dir, "gamma.bin", row);
  if (!h_g2 || !h_idx || !h_w || !h_pk || !h_sh || !h_gam) return 6;

  void *d_g2, *d_idx, *d_w, *d_pk, *d_sh, *d_out, *d_outp, *d_q, *d_s, *d_err, *d_gam, *d_ro,
      *d_nm;
  CHECK_HIP(hipMalloc(&d_g2, (size_t)P * row));
  CHECK_HIP(hipMalloc(&d_idx, slots * 4));
  CHECK_HIP(hipMalloc(&d_w, slots * 4));
  CHECK_HIP(hipMalloc(&d_pk, slots * 4));
  CHECK_HIP(hipMalloc(&d_sh, (size_t)T * row));
  CHECK_HIP(hipMalloc(&d_out, (size_t)T * row));
  CHECK_HIP(hipMalloc(&d_outp, (size_t)T * row));
  CHECK_HIP(hipMalloc(&d_q, (size_t)(T * H)));
  CHECK_HIP(hipMalloc(&d_s, (size_t)(T * (H / 128)) + 1));
  CHECK_HIP(hipMalloc(&d_err, 4));
  CHECK_HIP(hipMalloc(&d_gam, row));
  CHECK_HIP(hipMalloc(&d_ro, (size_t)T * row));
  CHECK_HIP(hipMalloc(&d_nm, (size_t)T * row));
  CHECK_HIP(hipMemcpy(d_gam, h_gam, row, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_g2, h_g2, (size_t)P * row, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_idx, h_idx, slots * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_w, h_w, slots * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_pk, h_pk, slots * 4, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_sh, h_sh, (size_t)T * row, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemset(d_err, 0, 4));

  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));
  bad |= expect(moe_finalize(d_g2, P, d_idx, d_w, NULL, d_sh, rsf, d_out, T, H, (int32_t)K,
                             d_err, stream), MOEF_OK, "moe_finalize fp32");
  bad |= expect(moe_finalize(d_g2, P, d_idx, NULL, d_pk, d_sh, rsf, d_outp, T, H, (int32_t)K,
                             d_err, stream), MOEF_OK, "moe_finalize packed");
  if (H % 128 == 0)
    bad |= expect(moe_finalize_quant_ue8m0(d_g2, P, d_idx, d_w, NULL, d_sh, rsf, d_q, d_s, T, H,
                                           (int32_t)K, d_err, stream),
                  MOEF_OK, "moe_finalize_quant_ue8m0");
  {
    const uint16_t* ranks[2] = {(const uint16_t*)d_out, (const uint16_t*)d_outp};
    bad |= expect(moe_allreduce_residual_rmsnorm(NULL, 2, d_sh, d_gam, 1e-6f, d_ro, d_nm, T, H,
                                                 stream),
                  MOEF_ERR_NULL_POINTER, "all-reduce without a rank array");
    bad |= expect(moe_allreduce_residual_rmsnorm(ranks, 0, d_sh, d_gam, 1e-6f, d_ro, d_nm, T, H,
                                                 stream),
                  MOEF_ERR_BAD_SHAPE, "all-reduce with no ranks");
    bad |= expect(moe_allreduce_residual_rmsnorm(ranks, 2, d_sh, d_gam, 1e-6f, d_ro, d_nm, T, H,
                                                 stream),
                  MOEF_OK, "moe_allreduce_residual_rmsnorm");
  }
  CHECK_HIP(hipStreamSynchronize(stream));
  if (bad) return 7;

  void* h_out = malloc((size_t)T * row);
  int32_t err = -1;
  CHECK_HIP(hipMemcpy(h_out, d_out, (size_t)T * row, hipMemcpyDeviceToHost));
  if (write_file(dir, "out.bin", h_out, (size_t)T * row)) return 8;
  CHECK_HIP(hipMemcpy(h_out, d_outp, (size_t)T * row, hipMemcpyDeviceToHost));
  if (write_file(dir, "out_packed.bin", h_out, (size_t)T * row)) return 8;
  if (H % 128 == 0) {
    CHECK_HIP(hipMemcpy(h_out, d_q, (size_t)(T * H), hipMemcpyDeviceToHost));
    if (write_file(dir, "q.bin", h_out, (size_t)(T * H))) return 8;
    CHECK_HIP(hipMemcpy(h_out, d_s, (size_t)(T * (H / 128)), hipMemcpyDeviceToHost));
    if (write_file(dir, "s.bin", h_out, (size_t)(T * (H / 128)))) return 8;
  }
  CHECK_HIP(hipMemcpy(&err, d_err, 4, hipMemcpyDeviceToHost));
  if (write_file(dir, "err.bin", &err, 4)) return 8;
  CHECK_HIP(hipMemcpy(h_out, d_ro, (size_t)T * row, hipMemcpyDeviceToHost));
  if (write_file(dir, "ro.bin", h_out, (size_t)T * row)) return 8;
  CHECK_HIP(hipMemcpy(h_out, d_nm, (size_t)T * row, hipMemcpyDeviceToHost));
  if (write_file(dir, "nm.bin", h_out, (size_t)T * row)) return 8;

  CHECK_HIP(hipStreamDestroy(stream));
  hipFree(d_g2); hipFree(d_idx); hipFree(d_w); hipFree(d_pk); hipFree(d_sh);
  hipFree(d_out); hipFree(d_outp); hipFree(d_q); hipFree(d_s); hipFree(d_err);
  hipFree(d_gam); hipFree(d_ro); hipFree(d_nm);
  free(h_g2); free(h_idx); free(h_w); free(h_pk); free(h_sh); free(h_gam); free(h_out);
  printf("abi_driver: ok\n");
  return 0;
}
