/* Host-only driver of libssd's argument checks, built with AddressSanitizer
 * and UndefinedBehaviorSanitizer on the host code (no GPU needed).  Every
 * call below has at least one invalid argument, so the library returns
 * before any HIP call; the workspace-size queries are host arithmetic.  Fake
 * device addresses are never dereferenced. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ssd.h"

#define FAKE ((void *)(uintptr_t)0x100000)
#define FAKE_F ((float *)(uintptr_t)0x100000)
#define MIS ((void *)(uintptr_t)0x100002)

static int failures = 0;

static void expect(const char *what, int got, int want) {
  const char *msg = ssd_last_error();
  if (got != want || !msg || !msg[0]) {
    printf("FAIL %s: got %d want %d (%s)\n", what, got, want, msg ? msg : "(null)");
    ++failures;
  }
}

static ssd_scan_args scan_ok(void) {
  ssd_scan_args a;
  memset(&a, 0, sizeof a);
  a.struct_size = sizeof a;
  a.dtype = SSD_DTYPE_BF16;
  a.batch = 2; a.seqlen = 300; a.nheads = 8; a.headdim = 64; a.dstate = 128; a.ngroups = 2; a.chunk_size = 128;
  a.x = FAKE; a.x_stride_token = 8 * 64; a.x_stride_batch = 300 * 8 * 64;
  a.B = FAKE; a.B_stride_token = 2 * 128; a.B_stride_batch = 300 * 2 * 128;
  a.C = FAKE; a.C_stride_token = 2 * 128; a.C_stride_batch = 300 * 2 * 128;
  a.dt = FAKE; a.dt_stride_token = 8; a.dt_stride_batch = 300 * 8;
  a.A = FAKE_F;
  a.y = FAKE; a.y_stride_token = 8 * 64; a.y_stride_batch = 300 * 8 * 64;
  return a;
}

int main(void) {
  if (ssd_version() < 1) { printf("FAIL version\n"); ++failures; }

  /* scan */
  expect("scan null", ssd_chunk_scan_fwd(NULL, NULL, 0, NULL), SSD_ERR_INVALID_ARG);
  ssd_scan_args s = scan_ok();
  if (ssd_chunk_scan_workspace_size(&s) == (size_t)-1) { printf("FAIL scan ws on valid args\n"); ++failures; }
  s.struct_size = 3;
  expect("scan struct_size", ssd_chunk_scan_fwd(&s, NULL, 0, NULL), SSD_ERR_INVALID_ARG);
  s = scan_ok(); s.ngroups = 3;
  expect("scan H % G", ssd_chunk_scan_fwd(&s, NULL, 0, NULL), SSD_ERR_INVALID_ARG);
  s = scan_ok(); s.headdim = 32;
  expect("scan headdim", ssd_chunk_scan_fwd(&s, NULL, 0, NULL), SSD_ERR_UNSUPPORTED);
  s = scan_ok(); s.x = MIS;
  expect("scan misaligned x", ssd_chunk_scan_fwd(&s, NULL, 0, NULL), SSD_ERR_MISALIGNED);
  s = scan_ok(); s.A = NULL;
  expect("scan no A", ssd_chunk_scan_fwd(&s, NULL, 0, NULL), SSD_ERR_INVALID_ARG);
  s = scan_ok(); s.seq_idx = (const int32_t *)FAKE; s.num_seqs = 0;
  expect("scan num_seqs", ssd_chunk_scan_fwd(&s, NULL, 0, NULL), SSD_ERR_INVALID_ARG);
  s = scan_ok(); s.headdim = 32;
  expect("noalloc headdim", ssd_chunk_scan_fwd_noalloc(&s, NULL), SSD_ERR_UNSUPPORTED);

  /* conv */
  ssd_conv_args c;
  memset(&c, 0, sizeof c);
  c.struct_size = sizeof c; c.dtype = SSD_DTYPE_BF16; c.batch = 1; c.seqlen = 10; c.channels = 64; c.width = 4;
  c.x = FAKE; c.x_stride_token = 64; c.x_stride_batch = 640; c.out = FAKE; c.out_stride_token = 64;
  c.out_stride_batch = 640; c.weight = NULL;
  expect("conv no weight", ssd_conv1d_silu(&c, NULL), SSD_ERR_INVALID_ARG);
  c.weight = FAKE_F; c.width = 3;
  expect("conv width", ssd_conv1d_silu(&c, NULL), SSD_ERR_UNSUPPORTED);
  expect("conv null", ssd_conv1d_silu(NULL, NULL), SSD_ERR_INVALID_ARG);

  /* conv + scan */
  ssd_conv_scan_args cs;
  memset(&cs, 0, sizeof cs);
  cs.struct_size = sizeof cs - 8;
  expect("conv_scan struct_size", ssd_conv_scan_fwd(&cs, NULL, 0, NULL), SSD_ERR_INVALID_ARG);
  if (ssd_conv_scan_workspace_size(&cs) != (size_t)-1) { printf("FAIL conv_scan ws on bad args\n"); ++failures; }

  /* decode */
  ssd_decode_args d;
  memset(&d, 0, sizeof d);
  d.struct_size = sizeof d; d.dtype = SSD_DTYPE_BF16; d.batch = 4; d.nheads = 8; d.headdim = 64; d.dstate = 128;
  d.ngroups = 3;
  expect("decode H % G", ssd_decode_step(&d, NULL), SSD_ERR_INVALID_ARG);
  expect("decode null", ssd_decode_step(NULL, NULL), SSD_ERR_INVALID_ARG);

  /* backward */
  ssd_scan_bwd_args b;
  memset(&b, 0, sizeof b);
  b.struct_size = sizeof b; b.dtype = SSD_DTYPE_BF16; b.batch = 1; b.seqlen = 64; b.nheads = 8; b.headdim = 64;
  b.dstate = 128; b.ngroups = 2;
  expect("bwd no A", ssd_chunk_scan_bwd(&b, NULL, 0, NULL), SSD_ERR_INVALID_ARG);
  b.A = FAKE_F; b.dA = FAKE_F; b.x = MIS; b.dt = FAKE; b.B = FAKE; b.C = FAKE; b.dy = FAKE; b.dx = FAKE;
  b.ddt = FAKE; b.dB = FAKE; b.dC = FAKE;
  expect("bwd misaligned", ssd_chunk_scan_bwd(&b, NULL, 0, NULL), SSD_ERR_MISALIGNED);
  b.x = FAKE;
  if (ssd_chunk_scan_bwd_workspace_size(&b) == (size_t)-1) { printf("FAIL bwd ws on valid args\n"); ++failures; }
  expect("bwd no workspace", ssd_chunk_scan_bwd(&b, NULL, 0, NULL), SSD_ERR_WORKSPACE_TOO_SMALL);

  /* gated norm */
  ssd_norm_args n;
  memset(&n, 0, sizeof n);
  n.struct_size = sizeof n;
  expect("norm zero dims", ssd_gated_rmsnorm(&n, NULL), SSD_ERR_INVALID_ARG);

  /* MIMO decode */
  ssd_mimo_decode_args m;
  memset(&m, 0, sizeof m);
  m.struct_size = sizeof m; m.dtype = SSD_DTYPE_BF16; m.batch = 2; m.nheads = 8; m.headdim = 64; m.dstate = 128;
  m.ngroups = 2; m.rank = 3;
  expect("mimo rank", ssd_decode_step_mimo(&m, NULL), SSD_ERR_UNSUPPORTED);

  /* linear */
  ssd_linear_args l;
  memset(&l, 0, sizeof l);
  l.struct_size = sizeof l; l.dtype = SSD_DTYPE_BF16; l.M = 16; l.N = 16; l.K = 100;
  expect("linear K", ssd_linear(&l, NULL), SSD_ERR_UNSUPPORTED);
  l.K = 64; l.N = 12;
  expect("linear N", ssd_linear(&l, NULL), SSD_ERR_UNSUPPORTED);

  printf("%s: %d failure(s)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
