/* A plain C99 caller of the libra C ABI (no HIP headers, no GPU): the header compiles
 * as C, the structs have the sizes the header states, and the host-side entry points
 * (version, status strings, *_validate, workspace queries) link and behave from C.
 * The data pointers are never dereferenced by validation, so aligned placeholders do. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ra.h"

static int failures = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static ra_tensor tensor4(uintptr_t addr, int dtype, int64_t a, int64_t b, int64_t c, int64_t d) {
  ra_tensor t;
  memset(&t, 0, sizeof t);
  t.data = (void *)addr;
  t.dtype = dtype;
  t.ndim = 4;
  t.shape[0] = a; t.shape[1] = b; t.shape[2] = c; t.shape[3] = d;
  t.stride[3] = 1; t.stride[2] = d; t.stride[1] = c * d; t.stride[0] = b * c * d;
  return t;
}

static ra_tensor tensor3(uintptr_t addr, int dtype, int64_t a, int64_t b, int64_t c) {
  ra_tensor t;
  memset(&t, 0, sizeof t);
  t.data = (void *)addr;
  t.dtype = dtype;
  t.ndim = 3;
  t.shape[0] = a; t.shape[1] = b; t.shape[2] = c;
  t.stride[2] = 1; t.stride[1] = c; t.stride[0] = b * c;
  return t;
}

int main(void) {
  const uintptr_t base = (uintptr_t)1 << 40;  /* placeholder device addresses, 16-aligned */
  ra_attn_params p;
  ra_tensor q, k, v, o, lse, bad;
  size_t ws_mha, ws_gqa;
  int s;

  CHECK(sizeof(ra_tensor) == 80);
  CHECK(sizeof(ra_attn_params) == RA_ATTN_PARAMS_SIZE_V2);
  CHECK(ra_version() == RA_VERSION);
  for (s = RA_OK; s >= RA_ERR_SCRATCH; --s) CHECK(ra_status_string(s) != NULL);
  CHECK(strcmp(ra_status_string(RA_OK), ra_status_string(RA_ERR_SHAPE)) != 0);

  memset(&p, 0, sizeof p);
  p.struct_size = sizeof p;
  p.causal = 1;
  p.num_chunks = 1;

  /* a GQA forward: 4 query heads over 2 key/value heads, 64 tokens, D = 128 */
  q = tensor4(base, RA_BF16, 1, 4, 64, 128);
  k = tensor4(base + 0x100000, RA_BF16, 1, 2, 64, 128);
  v = tensor4(base + 0x200000, RA_BF16, 1, 2, 64, 128);
  o = tensor4(base + 0x300000, RA_BF16, 1, 4, 64, 128);
  lse = tensor3(base + 0x400000, RA_F32, 1, 4, 64);
  CHECK(ra_attn_fwd_validate(&q, &k, &v, &p, &o, &lse) == RA_OK);
  CHECK(ra_attn_fwd_validate(NULL, &k, &v, &p, &o, &lse) == RA_ERR_NULL);

  bad = v;
  bad.dtype = RA_F32;
  CHECK(ra_attn_fwd_validate(&q, &k, &bad, &p, &o, &lse) == RA_ERR_DTYPE);
  bad = k;
  bad.shape[1] = 3; /* 4 query heads do not split over 3 key/value heads */
  CHECK(ra_attn_fwd_validate(&q, &bad, &v, &p, &o, &lse) == RA_ERR_SHAPE);
  bad = v;
  bad.data = (void *)(base + 0x200008); /* not 16-byte aligned */
  CHECK(ra_attn_fwd_validate(&q, &k, &bad, &p, &o, &lse) == RA_ERR_ALIGN);
  p.num_chunks = 0;
  CHECK(ra_attn_fwd_validate(&q, &k, &v, &p, &o, &lse) == RA_ERR_RANGE);
  p.num_chunks = 1;

  /* the backward's workspace: D_i rows, plus fp32 dK/dV partials with grouped heads */
  ws_gqa = ra_attn_bwd_workspace_size(&q, &k, &p);
  ws_mha = ra_attn_bwd_workspace_size(&q, &o, &p);
  CHECK(ws_mha == 4 * 64 * sizeof(float));
  CHECK(ws_gqa == ws_mha + 2 * 4 * 64 * 128 * sizeof(float));
  CHECK(ra_noalloc_scratch_bytes() > 0);

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("c abi ok\n");
  return 0;
}
