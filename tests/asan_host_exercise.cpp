// Host-layer exercise for the AddressSanitizer build (tests/test_asan_host.py):
// every entry point path of include/moe.h that runs without a GPU, over a
// sweep of valid and invalid configurations.  Exits non-zero on a wrong
// status; ASan aborts on any bad host memory access or leak.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>

#include "moe.h"

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expectation failed: %s (last error: %s)\n", \
              __FILE__, __LINE__, #cond, moe_last_error());            \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static moe_config_t base() {
  moe_config_t c;
  memset(&c, 0, sizeof(c));
  c.T = 2048; c.d_model = 4096; c.d_ff = 14336; c.n_experts = 8; c.top_k = 2;
  c.capacity_factor = 1.25; c.dtype = MOE_DTYPE_BF16;
  return c;
}

int main() {
  // the page's worked example and a sweep of shapes, factors and policies
  moe_config_t c = base();
  EXPECT(moe_check_config(&c) == MOE_OK);
  EXPECT(moe_capacity(&c) == 640);
  const int64_t Ts[] = {0, 1, 7, 64, 129, 2048, 16384, 100003};
  const int Es[] = {1, 2, 8, 65, 160, 256};
  const double cfs[] = {0.0, -1.0, 1e-300, 5e-324, 0.3, 1.0, 1.1, 1.25, 2.0 / 3.0, 999999.0};
  for (int64_t T : Ts)
    for (int E : Es)
      for (int k : {1, 2, 6})
        for (double cf : cfs)
          for (int pol = 0; pol < 3; ++pol)
            for (int S : {0, 2}) {
              if (k > E) continue;
              moe_config_t x = base();
              x.T = T; x.n_experts = E; x.top_k = k; x.capacity_factor = cf;
              x.overflow = pol; x.n_shared = S;
              x.d_model = E > 100 ? 5120 : 4096;
              x.d_ff = E > 100 ? 1536 : 14336;
              x.weight_layout = (T & 1) ? MOE_WEIGHTS_PACKED : MOE_WEIGHTS_ROW_MAJOR;
              EXPECT(moe_check_config(&x) == MOE_OK);
              const size_t ws = moe_workspace_size(&x);
              EXPECT(T == 0 || ws > 0);
              const int64_t C = moe_capacity(&x);
              EXPECT(C >= 0);
              if (cf > 0.0 && T > 0) EXPECT(C >= 1);
              size_t w13 = 0, w2 = 0;
              EXPECT(moe_packed_weight_bytes(&x, &w13, &w2) == MOE_OK && w13 > 0 && w2 > 0);
            }
  // invalid configurations: a status and a message, never a crash
  moe_config_t bad = base();
  bad.top_k = 9;
  EXPECT(moe_check_config(&bad) == MOE_EINVAL && strlen(moe_last_error()) > 0);
  EXPECT(moe_workspace_size(&bad) == 0 && moe_capacity(&bad) == -1);
  bad = base(); bad.capacity_factor = NAN;
  EXPECT(moe_check_config(&bad) == MOE_EINVAL);
  bad = base(); bad.T = int64_t(1) << 40;
  EXPECT(moe_check_config(&bad) == MOE_EINVAL);
  bad = base(); bad.d_model = 100;
  EXPECT(moe_check_config(&bad) == MOE_EUNSUPPORTED);
  bad = base(); bad.out_fp32 = 3;
  EXPECT(moe_check_config(&bad) == MOE_EINVAL);
  EXPECT(moe_check_config(nullptr) == MOE_EINVAL);
  // calls that return before any GPU work: empty batches, argument checks
  moe_config_t e = base();
  e.T = 0;
  moe_stats_t st;
  memset(&st, 0, sizeof(st));
  int64_t counts[8], kept[8];
  st.counts = counts; st.kept = kept;
  EXPECT(moe_forward(nullptr, nullptr, nullptr, nullptr, nullptr, &e, nullptr, &st) == MOE_OK);
  EXPECT(st.dropped == 0 && st.aux_loss == 0.0 && counts[0] == 0);
  EXPECT(moe_forward(nullptr, nullptr, nullptr, nullptr, nullptr, &c, nullptr, nullptr) == MOE_EINVAL);
  int dummy = 0;
  EXPECT(moe_forward(&dummy, &dummy, &dummy, &dummy, &dummy, &c, &dummy, nullptr) == MOE_EWORKSPACE);
  EXPECT(moe_forward_noalloc(&dummy, &dummy, &dummy, &dummy, &dummy, &c, &dummy, nullptr) ==
         MOE_EWORKSPACE);
  EXPECT(moe_route_logits(nullptr, &c, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                          nullptr) == MOE_EINVAL);
  double aux = -1.0;
  EXPECT(moe_aux_loss(nullptr, nullptr, &e, &aux) == MOE_OK && aux == 0.0);
  EXPECT(moe_router_backward(nullptr, nullptr, nullptr, NAN, 0.0, &c, nullptr, nullptr, nullptr,
                             nullptr) == MOE_EINVAL);
  // training-side helpers
  EXPECT(moe_entropy_coef(0, 101, 0.5, 0.01) == 0.5);
  EXPECT(fabs(moe_entropy_coef(100, 101, 0.5, 0.01) - 0.01) < 1e-15);
  double vals[1000], slope = 0.0, mean = 0.0;
  for (int i = 0; i < 1000; ++i) vals[i] = 3.0 - 0.25 * i;
  EXPECT(moe_lb_trend(vals, 1000, &slope, &mean) == MOE_OK && fabs(slope + 0.25) < 1e-12);
  EXPECT(moe_lb_trend(vals, 1, &slope, &mean) == MOE_EINVAL);
  EXPECT(moe_lb_trend(nullptr, 5, &slope, &mean) == MOE_EINVAL);
  // per-kernel timing bookkeeping without any launch
  EXPECT(moe_timing_only("ffn1_swiglu,combine") == MOE_OK);
  EXPECT(moe_timing_only(nullptr) == MOE_OK);
  EXPECT(moe_timing_reset() == MOE_OK);
  char names[64 * 4];
  int64_t launches[4];
  double ms[4];
  EXPECT(moe_timing_read(names, launches, ms, 4) == 0);
  printf("asan host exercise: %d failures\n", failures);
  return failures ? 1 : 0;
}
