/* c_driver.c -- drives the library through its C ABI alone (no Python).
 *
 * Reads a job file, runs spec compile, descriptor size/init/build, forward
 * and backward on the default stream, and writes every output to a result
 * file.  The GPU test that builds and runs this program compares the results
 * with the Python binding's on the same inputs.
 *
 * Job file (little-endian):
 *   int32 B, H, N, d, n_scalars, seg_cap, n_refs, fwd_q, fwd_k, bwd_k, bwd_q, spec_len
 *   char  spec[spec_len]
 *   int32 scalars[B*n_scalars], seg_bounds[B*(seg_cap+1)], n_seg[B], refs[B*seg_cap*n_refs]
 *   bf16  q, k, v, dO: [B][H][N][d] each
 *   int32 has_bad; if 1, a second metadata set of the same sizes (scalars,
 *         seg_bounds, n_seg, refs) that the device is to flag as invalid
 * Result file: bf16 o, dq, dk, dv; fp32 lse[B][H][N]; the descriptor bytes;
 * with has_bad also uint32 flags, uint32 per-sample error words[B] (from
 * cm_desc_errors) and the second descriptor's bytes (from cm_desc_download).
 * Exit status 0 on success; otherwise the failing call is printed.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "compilemask.h"

#define CHECK_CM(call)                                                                       \
  do {                                                                                       \
    cm_status st_ = (call);                                                                  \
    if (st_ != CM_OK) {                                                                      \
      fprintf(stderr, "%s: %s (%s)\n", #call, cm_status_str(st_), cm_last_error());          \
      return 1;                                                                              \
    }                                                                                        \
  } while (0)
#define CHECK_HIP(call)                                                                      \
  do {                                                                                       \
    hipError_t e_ = (call);                                                                  \
    if (e_ != hipSuccess) {                                                                  \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));                             \
      return 1;                                                                              \
    }                                                                                        \
  } while (0)

static int read_all(FILE* f, void* dst, size_t bytes) { return fread(dst, 1, bytes, f) == bytes ? 0 : 1; }

static void* upload(const void* host, size_t bytes) {
  void* dev = NULL;
  if (!bytes) return NULL;
  if (hipMalloc(&dev, bytes) != hipSuccess) return NULL;
  if (hipMemcpy(dev, host, bytes, hipMemcpyHostToDevice) != hipSuccess) return NULL;
  return dev;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s JOB RESULT\n", argv[0]);
    return 2;
  }
  FILE* f = fopen(argv[1], "rb");
  if (!f) return 2;
  int32_t h[12];
  if (read_all(f, h, sizeof(h))) return 2;
  const int32_t B = h[0], H = h[1], N = h[2], d = h[3], ns = h[4], cap = h[5], nr = h[6];
  const cm_tiles tiles = {h[7], h[8], h[9], h[10]};
  char* text = (char*)calloc((size_t)h[11] + 1, 1);
  if (read_all(f, text, (size_t)h[11])) return 2;
  const size_t n_sc = (size_t)B * ns, n_sb = (size_t)B * (cap + 1), n_rf = (size_t)B * cap * nr;
  int32_t* meta = (int32_t*)malloc((n_sc + n_sb + B + n_rf + 1) * 4);
  if (read_all(f, meta, (n_sc + n_sb + B + n_rf) * 4)) return 2;
  const size_t elems = (size_t)B * H * N * d, tbytes = elems * 2, lbytes = (size_t)B * H * N * 4;
  unsigned char* inputs = (unsigned char*)malloc(4 * tbytes);
  if (read_all(f, inputs, 4 * tbytes)) return 2;
  int32_t has_bad = 0;
  int32_t* bad = NULL;
  if (fread(&has_bad, 4, 1, f) != 1) has_bad = 0;
  if (has_bad) {
    bad = (int32_t*)malloc((n_sc + n_sb + B + n_rf + 1) * 4);
    if (read_all(f, bad, (n_sc + n_sb + B + n_rf) * 4)) return 2;
  }
  fclose(f);

  cm_spec* spec = NULL;
  CHECK_CM(cm_spec_compile(text, &spec));
  size_t dbytes = 0;
  CHECK_CM(cm_desc_size(spec, B, N, cap, &tiles, &dbytes));
  void* dbuf = NULL;
  CHECK_HIP(hipMalloc(&dbuf, dbytes));  /* hipMalloc returns 256-byte aligned memory */
  cm_desc* desc = NULL;
  CHECK_CM(cm_desc_init(spec, B, N, cap, &tiles, dbuf, dbytes, &desc));

  cm_metadata md;
  md.scalars = (const int32_t*)upload(meta, n_sc * 4);
  md.seg_bounds = (const int32_t*)upload(meta + n_sc, n_sb * 4);
  md.n_seg = (const int32_t*)upload(meta + n_sc + n_sb, (size_t)B * 4);
  md.refs = (const int32_t*)upload(meta + n_sc + n_sb + B, n_rf * 4);
  md.n_scalars = ns;
  md.n_refs = nr;
  md.cu_seqlens = NULL;

  void *q = upload(inputs, tbytes), *k = upload(inputs + tbytes, tbytes);
  void *v = upload(inputs + 2 * tbytes, tbytes), *dO = upload(inputs + 3 * tbytes, tbytes);
  void *o, *dq, *dk, *dv, *ws;
  float* lse;
  cm_attn_args args;
  memset(&args, 0, sizeof(args));
  args.B = B; args.H = H; args.N = N; args.d = d;  /* contiguous strides, scale 1/sqrt(d) */
  size_t wbytes = 0;
  CHECK_CM(cm_attn_bwd_workspace(&args, &wbytes));
  CHECK_HIP(hipMalloc(&o, tbytes));
  CHECK_HIP(hipMalloc(&dq, tbytes));
  CHECK_HIP(hipMalloc(&dk, tbytes));
  CHECK_HIP(hipMalloc(&dv, tbytes));
  CHECK_HIP(hipMalloc((void**)&lse, lbytes));
  CHECK_HIP(hipMalloc(&ws, wbytes));

  CHECK_CM(cm_build_descriptor(spec, &md, desc, NULL));
  CHECK_CM(cm_attn_fwd(&args, q, k, v, desc, o, lse, NULL));
  CHECK_CM(cm_attn_bwd(&args, q, k, v, o, lse, dO, desc, dq, dk, dv, ws, wbytes, NULL));
  CHECK_HIP(hipDeviceSynchronize());

  unsigned char* out = (unsigned char*)malloc(4 * tbytes + lbytes + dbytes);
  void* srcs[4] = {o, dq, dk, dv};
  for (int i = 0; i < 4; ++i) CHECK_HIP(hipMemcpy(out + i * tbytes, srcs[i], tbytes, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(out + 4 * tbytes, lse, lbytes, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(out + 4 * tbytes + lbytes, dbuf, dbytes, hipMemcpyDeviceToHost));
  FILE* g = fopen(argv[2], "wb");
  if (!g || fwrite(out, 1, 4 * tbytes + lbytes + dbytes, g) != 4 * tbytes + lbytes + dbytes) return 3;

  if (has_bad) {
    /* the same descriptor rebuilt from metadata the device must reject */
    cm_metadata bmd = md;
    bmd.scalars = (const int32_t*)upload(bad, n_sc * 4);
    bmd.seg_bounds = (const int32_t*)upload(bad + n_sc, n_sb * 4);
    bmd.n_seg = (const int32_t*)upload(bad + n_sc + n_sb, (size_t)B * 4);
    bmd.refs = (const int32_t*)upload(bad + n_sc + n_sb + B, n_rf * 4);
    CHECK_CM(cm_build_descriptor(spec, &bmd, desc, NULL));
    uint32_t flags = 0;
    int32_t n_err = 0;
    uint32_t* per = (uint32_t*)calloc((size_t)B, 4);
    CHECK_CM(cm_desc_errors(desc, &flags, per, &n_err, NULL));
    if (n_err != B) {
      fprintf(stderr, "cm_desc_errors reported %d sample words, expected %d\n", n_err, B);
      return 1;
    }
    unsigned char* words = (unsigned char*)malloc(dbytes);
    if (cm_desc_download(desc, words, dbytes - 4, NULL) != CM_ERR_SIZE) {
      fprintf(stderr, "cm_desc_download accepted a buffer smaller than the descriptor\n");
      return 1;
    }
    CHECK_CM(cm_desc_download(desc, words, dbytes, NULL));
    if (fwrite(&flags, 4, 1, g) != 1 || fwrite(per, 4, (size_t)B, g) != (size_t)B || fwrite(words, 1, dbytes, g) != dbytes)
      return 3;
    printf("c_driver: invalid metadata flagged 0x%x\n", flags);
  }
  fclose(g);

  cm_desc_free(desc);
  cm_spec_free(spec);
  printf("c_driver ok: %d x %d x %d x %d, descriptor %zu bytes\n", B, H, N, d, dbytes);
  return 0;
}
