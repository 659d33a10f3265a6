// Host-side argument-check driver for the sanitizer test: calls every entry point
// of include/hla.h over a grid of shapes, dtype codes and arguments, each call
// carrying at least one invalid argument or an empty tensor, so that validation
// returns before any HIP call and no GPU is needed. Built against a copy of the
// library whose host code carries AddressSanitizer and UndefinedBehaviorSanitizer;
// a sanitizer report aborts the process. Exits 0 after printing the call count
// when every call returned the status the grid expects.
#include <stdint.h>
#include <stdio.h>
#include <math.h>
#include <stdlib.h>

#include "../../include/hla.h"

static void* const FAKE = (void*)0x10000;  // 16-byte aligned, never dereferenced
static void* const ODD = (void*)0x10008;   // 8-byte aligned only
static long calls = 0, failures = 0;

static void expect(int got, int bad_expected, const char* what, const hla_dims* d) {
  ++calls;
  // bad_expected: the call must not succeed (it carried an invalid argument)
  if (bad_expected && got == HLA_OK) {
    if (failures++ < 20)
      fprintf(stderr, "%s returned HLA_OK for B=%lld H=%lld N=%lld D=%lld in=%d out=%d\n", what,
              (long long)d->B, (long long)d->H, (long long)d->N, (long long)d->D, d->in_dtype,
              d->out_dtype);
  }
  if (got < HLA_OK || got > HLA_ERR_HIP) {
    if (failures++ < 20) fprintf(stderr, "%s returned unknown status %d\n", what, got);
  }
  if (!hla_status_str(got)) ++failures;
}

int main(void) {
  const int64_t dimv[] = {-1, 0, 1, 7, 256, 19320, (int64_t)1 << 31, (int64_t)1 << 40, INT64_MAX};
  const int64_t dv[] = {-1, 0, 16, 32, 64, 96, 128, 256};
  const int32_t dtv[] = {-1, HLA_F32, HLA_BF16, HLA_FP8_E4M3, 3};
  const size_t ndim = sizeof(dimv) / sizeof(dimv[0]), nd = sizeof(dv) / sizeof(dv[0]),
               ndt = sizeof(dtv) / sizeof(dtv[0]);
  const void* ptrs[4] = {FAKE, FAKE, FAKE, FAKE};
  const int32_t kinds[2] = {HLA_LAYER_LINEAR, HLA_LAYER_SOFTMAX};
  const void* sums[2] = {FAKE, FAKE};
  int variant = 0;
  for (size_t ib = 0; ib < ndim; ++ib)
    for (size_t ih = 0; ih < ndim; ++ih)
      for (size_t in = 0; in < ndim; ++in)
        for (size_t id = 0; id < nd; ++id)
          for (size_t ii = 0; ii < ndt; ++ii)
            for (size_t io = 0; io < ndt; ++io) {
              hla_dims d = {dimv[ib], dimv[ih], dimv[in], dv[id], dtv[ii], dtv[io]};
              // workspace queries are pure and never fail
              (void)hla_linear_workspace_bytes(&d);
              (void)hla_softmax_anchor_workspace_bytes(&d);
              // the one invalid argument of this call (rotates over the kinds); a
              // call on a non-empty tensor must then be refused (an empty one may
              // return HLA_OK: its pointers are not read)
              const int bad = variant++ % 6;
              const int ne = d.B > 0 && d.H > 0 && d.N > 0;
              void* q = bad == 0 ? NULL : FAKE;
              void* out = bad == 1 ? ODD : FAKE;
              const float eps = bad == 2 ? -1.0f : 1e-6f;
              const float scale = bad == 2 ? 0.0f : 0.1f;
              const int acc = bad == 3 ? 2 : 0;
              const size_t wsb = bad == 4 ? 1 : ((size_t)1 << 62);
              void* ws = bad == 5 ? ODD : FAKE;
              expect(hla_linear_fwd(&d, q, FAKE, FAKE, FAKE, out, acc, eps, ws, wsb, NULL), ne,
                     "hla_linear_fwd", &d);
              expect(hla_linear_write_gated_fwd(&d, q, FAKE, FAKE, FAKE, bad == 5 ? NULL : FAKE, out,
                                                acc, eps, ws, wsb, NULL),
                     ne, "hla_linear_write_gated_fwd", &d);
              // the allocation-free call has no workspace: a tiny N keeps it
              // within the scratch limit, so its invalid argument is q, out,
              // eps or accumulate
              const int nb = variant % 4;
              expect(hla_linear_fwd_noalloc(&d, nb == 0 ? NULL : FAKE, FAKE, FAKE, FAKE,
                                            nb == 1 ? ODD : FAKE, nb == 3 ? 2 : 0,
                                            nb == 2 ? NAN : 1e-6f, NULL),
                     ne, "hla_linear_fwd_noalloc", &d);
              expect(hla_softmax_anchor_fwd(&d, q, FAKE, FAKE, FAKE, out, acc, scale, ws, wsb, NULL),
                     ne, "hla_softmax_anchor_fwd", &d);
              expect(hla_softmax_anchor_fp8p_fwd(&d, q, FAKE, FAKE, FAKE, out, acc, scale, ws, wsb,
                                                 NULL),
                     ne, "hla_softmax_anchor_fp8p_fwd", &d);
              const void* qa[2] = {bad == 0 ? NULL : FAKE, FAKE};
              expect(hla_hybrid_stack_fwd(&d, bad == 3 ? 0 : 2, kinds, qa, ptrs, ptrs, ptrs, out, eps,
                                          scale, ws, wsb, NULL),
                     ne, "hla_hybrid_stack_fwd", &d);
              const void* sa[2] = {bad == 0 ? NULL : FAKE, FAKE};
              expect(hla_attnres_route_fwd(&d, bad == 3 ? 17 : 2, bad == 4 ? NULL : sa,
                                           bad == 2 ? NULL : FAKE, bad == 5 ? ODD : FAKE, out, NULL),
                     ne, "hla_attnres_route_fwd", &d);
              // an empty tensor with otherwise valid arguments returns HLA_OK
              // without touching the null pointers
              hla_dims e = d;
              e.N = 0;
              if (e.B >= 0 && e.H >= 0 && e.D > 0) {
                (void)hla_linear_fwd(&e, NULL, NULL, NULL, NULL, NULL, 0, 1e-6f, NULL, 0, NULL);
                (void)hla_softmax_anchor_fwd(&e, NULL, NULL, NULL, NULL, NULL, 0, 0.1f, NULL, 0, NULL);
                (void)hla_linear_fwd_noalloc(&e, NULL, NULL, NULL, NULL, NULL, 0, 1e-6f, NULL);
                calls += 3;
              }
            }
  (void)sums;
  for (int s = -3; s < 12; ++s) (void)hla_status_str(s);
  printf("calls %ld failures %ld abi %d\n", calls, failures, hla_abi_version());
  return failures ? 1 : 0;
}
