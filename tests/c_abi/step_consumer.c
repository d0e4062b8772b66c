/*
 * A C program that uses the library through include/dit_attn.h only: device buffers from
 * hipMalloc, its own stream, no Python and no PyTorch.  It runs a sequence of selective
 * steps (dit_attn_partitioned) on inputs read from a file and writes the outputs of every
 * step to another file, so that a test can compare them with the Python binding's and with
 * the oracle.
 *
 * Input file (little endian):
 *   int32 B, S_q, S_kv, H, D, n_qb, P, steps
 *   int32 q_offsets[n_qb + 1], kv_offsets[P + 1], local_part[n_qb]
 *   per step: uint8 recompute[n_qb * P], uint8 want_importance, uint8 want_delta,
 *             uint16 q[B S_q H D], k[B S_kv H D], v[B S_kv H D]   (bf16 bit patterns)
 * Output file, per step:
 *   int32 status, uint8 did_delta,
 *   uint16 out[B S_q H D], float lse[B H S_q], float importance[B n_qb P], float delta[B n_qb]
 *   (importance and delta are zero when not requested or not computed)
 *
 *   step_consumer <input> <output>
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "dit_attn.h"

#define CHECK_HIP(x)                                                                    \
  do {                                                                                  \
    hipError_t e_ = (x);                                                                \
    if (e_ != hipSuccess) {                                                             \
      fprintf(stderr, "%s:%d: %s -> %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
      exit(3);                                                                          \
    }                                                                                   \
  } while (0)

static void read_all(FILE *f, void *dst, size_t bytes) {
  if (bytes && fread(dst, 1, bytes, f) != bytes) {
    fprintf(stderr, "input file too short\n");
    exit(2);
  }
}

static void write_all(FILE *f, const void *src, size_t bytes) {
  if (bytes && fwrite(src, 1, bytes, f) != bytes) {
    fprintf(stderr, "cannot write output\n");
    exit(2);
  }
}

static void *host_alloc(size_t bytes) {
  void *p = malloc(bytes ? bytes : 1);
  if (!p) {
    fprintf(stderr, "out of host memory\n");
    exit(2);
  }
  return p;
}

static void *dev_alloc(size_t bytes) {
  void *p = NULL;
  CHECK_HIP(hipMalloc(&p, bytes ? bytes : 1));
  return p;
}

int main(int argc, char **argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s <input> <output>\n", argv[0]);
    return 2;
  }
  FILE *in = fopen(argv[1], "rb");
  FILE *out = fopen(argv[2], "wb");
  if (!in || !out) {
    fprintf(stderr, "cannot open files\n");
    return 2;
  }
  int32_t hdr[8];
  read_all(in, hdr, sizeof(hdr));
  const int B = hdr[0], S_q = hdr[1], S_kv = hdr[2], H = hdr[3], D = hdr[4], n_qb = hdr[5], P = hdr[6];
  const int steps = hdr[7];
  if (B < 1 || S_q < 1 || S_kv < 0 || H < 1 || n_qb < 1 || n_qb > DIT_MAX_BLOCKS || P < 1 ||
      P > DIT_MAX_PARTITIONS || steps < 1) {
    fprintf(stderr, "bad header\n");
    return 2;
  }
  int32_t *q_offsets = host_alloc(sizeof(int32_t) * (n_qb + 1));
  int32_t *kv_offsets = host_alloc(sizeof(int32_t) * (P + 1));
  int32_t *local_part = host_alloc(sizeof(int32_t) * n_qb);
  read_all(in, q_offsets, sizeof(int32_t) * (n_qb + 1));
  read_all(in, kv_offsets, sizeof(int32_t) * (P + 1));
  read_all(in, local_part, sizeof(int32_t) * n_qb);

  const size_t nq = (size_t)B * S_q * H * D, nkv = (size_t)B * S_kv * H * D;
  const size_t nrh = (size_t)B * S_q * H;
  uint8_t *recompute = host_alloc((size_t)n_qb * P);
  uint8_t *valid = host_alloc((size_t)n_qb * P);
  memset(valid, 0, (size_t)n_qb * P);
  uint16_t *h_q = host_alloc(nq * 2), *h_k = host_alloc(nkv * 2), *h_v = host_alloc(nkv * 2);
  uint16_t *h_out = host_alloc(nq * 2);
  float *h_lse = host_alloc(nrh * 4);
  float *h_imp = host_alloc((size_t)B * n_qb * P * 4);
  float *h_delta = host_alloc((size_t)B * n_qb * 4);

  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));
  void *d_q = dev_alloc(nq * 2), *d_k = dev_alloc(nkv * 2), *d_v = dev_alloc(nkv * 2);
  void *d_cache_o = dev_alloc((size_t)P * nq * 2);
  float *d_cache_lse = dev_alloc((size_t)P * nrh * 4);
  void *d_out = dev_alloc(nq * 2);
  float *d_lse = dev_alloc(nrh * 4);
  float *d_imp = dev_alloc((size_t)B * n_qb * P * 4);
  float *d_delta = dev_alloc((size_t)B * n_qb * 4);
  const size_t ws_bytes = dit_attn_workspace_bytes(B, S_q, H, D, n_qb, P);
  if (ws_bytes == 0) {
    fprintf(stderr, "dit_attn_workspace_bytes rejected the sizes\n");
    return 2;
  }
  void *d_ws = dev_alloc(ws_bytes);

  for (int t = 0; t < steps; ++t) {
    uint8_t flags[2];
    read_all(in, recompute, (size_t)n_qb * P);
    read_all(in, flags, 2);
    read_all(in, h_q, nq * 2);
    read_all(in, h_k, nkv * 2);
    read_all(in, h_v, nkv * 2);
    CHECK_HIP(hipMemcpyAsync(d_q, h_q, nq * 2, hipMemcpyHostToDevice, stream));
    CHECK_HIP(hipMemcpyAsync(d_k, h_k, nkv * 2, hipMemcpyHostToDevice, stream));
    CHECK_HIP(hipMemcpyAsync(d_v, h_v, nkv * 2, hipMemcpyHostToDevice, stream));
    /* the local change needs a state in every local slot */
    int did_delta = flags[1] != 0;
    for (int i = 0; i < n_qb; ++i)
      if (!valid[i * P + local_part[i]]) did_delta = 0;
    const int32_t status = dit_attn_partitioned(
        d_q, d_k, d_v, B, S_q, S_kv, H, D, q_offsets, n_qb, kv_offsets, P, local_part, recompute, valid,
        d_cache_o, d_cache_lse, d_out, d_lse, 0.0f, flags[0] ? d_imp : NULL, did_delta ? d_delta : NULL, d_ws,
        ws_bytes, (void *)stream);
    if (status != DIT_OK) fprintf(stderr, "step %d: %s\n", t, dit_status_string(status));
    memset(h_imp, 0, (size_t)B * n_qb * P * 4);
    memset(h_delta, 0, (size_t)B * n_qb * 4);
    CHECK_HIP(hipMemcpyAsync(h_out, d_out, nq * 2, hipMemcpyDeviceToHost, stream));
    CHECK_HIP(hipMemcpyAsync(h_lse, d_lse, nrh * 4, hipMemcpyDeviceToHost, stream));
    if (flags[0]) CHECK_HIP(hipMemcpyAsync(h_imp, d_imp, (size_t)B * n_qb * P * 4, hipMemcpyDeviceToHost, stream));
    if (did_delta) CHECK_HIP(hipMemcpyAsync(h_delta, d_delta, (size_t)B * n_qb * 4, hipMemcpyDeviceToHost, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    if (status == DIT_OK)
      for (int e = 0; e < n_qb * P; ++e) valid[e] |= recompute[e];
    const uint8_t dd = (uint8_t)did_delta;
    write_all(out, &status, sizeof(status));
    write_all(out, &dd, 1);
    write_all(out, h_out, nq * 2);
    write_all(out, h_lse, nrh * 4);
    write_all(out, h_imp, (size_t)B * n_qb * P * 4);
    write_all(out, h_delta, (size_t)B * n_qb * 4);
  }
  CHECK_HIP(hipFree(d_q));
  CHECK_HIP(hipFree(d_k));
  CHECK_HIP(hipFree(d_v));
  CHECK_HIP(hipFree(d_cache_o));
  CHECK_HIP(hipFree(d_cache_lse));
  CHECK_HIP(hipFree(d_out));
  CHECK_HIP(hipFree(d_lse));
  CHECK_HIP(hipFree(d_imp));
  CHECK_HIP(hipFree(d_delta));
  CHECK_HIP(hipFree(d_ws));
  CHECK_HIP(hipStreamDestroy(stream));
  fclose(in);
  if (fclose(out) != 0) return 2;
  return 0;
}
