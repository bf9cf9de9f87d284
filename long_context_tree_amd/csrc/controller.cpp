// Draft-depth controller (host code): the closed-form choice of the next draft length from an
// online acceptance rate and an online draft/target cost ratio ("Adaptive Speculative Decoding",
// section "The controller"), with the long-context shallow starting depth of the DiffSpec plugin
// ("DiffSpec: Accelerating Long Sequence Generation with Differential Speculative Decoding",
// sections "Architecture" and "Configuration").
#include <cmath>
#include <cstdio>
#include <string>

#include "spec_internal.h"

namespace spec {
int host_fail(int status, const char* what);
}

namespace {

bool finite_in(double x, double lo, double hi) { return std::isfinite(x) && x >= lo && x <= hi; }

}  // namespace

extern "C" {

double spec_controller_speedup(double alpha, double cost_ratio, int32_t k) {
  if (!finite_in(alpha, 0.0, 1.0) || !(cost_ratio >= 0.0) || !std::isfinite(cost_ratio) || k < 0) return 0.0;
  // expected tokens per round: 1 + a + ... + a^k
  double tokens = 0.0, ap = 1.0;
  for (int32_t i = 0; i <= k; ++i) {
    tokens += ap;
    ap *= alpha;
  }
  return tokens / ((double)(k + 1) * cost_ratio + 1.0);
}

int32_t spec_controller_choose(double alpha, double cost_ratio, int32_t k_max) {
  if (k_max < 1 || !finite_in(alpha, 0.0, 1.0) || !(cost_ratio > 0.0) || !std::isfinite(cost_ratio)) return 0;
  int32_t best = 1;
  double best_v = spec_controller_speedup(alpha, cost_ratio, 1);
  for (int32_t k = 2; k <= k_max; ++k) {
    const double v = spec_controller_speedup(alpha, cost_ratio, k);
    if (v > best_v) {
      best_v = v;
      best = k;
    }
  }
  return best;
}

int spec_controller_init(spec_depth_controller* ctl, int32_t k_max, double alpha0, double cost_ratio0,
                         double alpha_decay, double cost_decay, int64_t ctx_len, int64_t long_ctx_threshold,
                         int32_t long_ctx_depth) {
  if (!ctl) return spec::host_fail(SPEC_ERR_INVALID_ARGUMENT, "ctl: NULL");
  if (k_max < 1) return spec::host_fail(SPEC_ERR_INVALID_ARGUMENT, "k_max: must be >= 1");
  if (!finite_in(alpha0, 0.0, 1.0)) return spec::host_fail(SPEC_ERR_INVALID_ARGUMENT, "alpha0: must be in [0, 1]");
  if (!(cost_ratio0 > 0.0) || !std::isfinite(cost_ratio0)) return spec::host_fail(SPEC_ERR_INVALID_ARGUMENT, "cost_ratio0: must be > 0");
  if (!(alpha_decay > 0.0) || !(alpha_decay <= 1.0)) return spec::host_fail(SPEC_ERR_INVALID_ARGUMENT, "alpha_decay: must be in (0, 1]");
  if (!(cost_decay > 0.0) || !(cost_decay <= 1.0)) return spec::host_fail(SPEC_ERR_INVALID_ARGUMENT, "cost_decay: must be in (0, 1]");
  if (long_ctx_depth < 1) return spec::host_fail(SPEC_ERR_INVALID_ARGUMENT, "long_ctx_depth: must be >= 1");
  ctl->alpha = alpha0;
  ctl->cost_ratio = cost_ratio0;
  ctl->alpha_decay = alpha_decay;
  ctl->cost_decay = cost_decay;
  ctl->k_max = k_max;
  ctl->rounds = 0;
  ctl->k = (long_ctx_threshold > 0 && ctx_len >= long_ctx_threshold)
               ? (long_ctx_depth < k_max ? long_ctx_depth : k_max)
               : spec_controller_choose(alpha0, cost_ratio0, k_max);
  return spec::host_fail(SPEC_OK, nullptr);
}

int spec_controller_update(spec_depth_controller* ctl, int32_t drafted, int32_t accepted, double t_draft,
                           double t_target) {
  if (!ctl) return spec::host_fail(SPEC_ERR_INVALID_ARGUMENT, "ctl: NULL");
  if (drafted < 0 || accepted < 0 || accepted > drafted)
    return spec::host_fail(SPEC_ERR_INVALID_ARGUMENT, "drafted / accepted: need 0 <= accepted <= drafted");
  if (!(t_target > 0.0) || !std::isfinite(t_target)) return spec::host_fail(SPEC_ERR_INVALID_ARGUMENT, "t_target: must be > 0");
  if (!(t_draft >= 0.0) || !std::isfinite(t_draft)) return spec::host_fail(SPEC_ERR_INVALID_ARGUMENT, "t_draft: must be >= 0");
  double a = ctl->alpha;
  const double w = ctl->alpha_decay;
  for (int32_t i = 0; i < accepted; ++i) a = (1.0 - w) * a + w * 1.0;
  if (accepted < drafted) a = (1.0 - w) * a;             // the first rejected draft
  ctl->alpha = a;
  if (t_draft > 0.0) ctl->cost_ratio = (1.0 - ctl->cost_decay) * ctl->cost_ratio + ctl->cost_decay * (t_draft / t_target);
  ctl->rounds += 1;
  ctl->k = spec_controller_choose(ctl->alpha, ctl->cost_ratio, ctl->k_max);
  return spec::host_fail(SPEC_OK, nullptr);
}

}  // extern "C"
