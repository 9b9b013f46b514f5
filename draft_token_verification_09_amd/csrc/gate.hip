// Acceptance telemetry and the adaptive speculation gate (host code only).
//
// "Breaking the Memory Bandwidth Wall: 3.42x Generation Speedup with EAGLE Speculative
// Decoding" (acefleet.dev), "Closed-Loop Real-Time Adaptive Gating": a temperature
// limit of 0.70 and a per-tenant exponential moving average of the acceptance rate
// whose drop below 0.55 trips a circuit breaker.  The readings of what the page leaves
// open (EMA start and weight, cooldown, trial) are stated with the declarations.
#include <cmath>
#include <mutex>
#include <new>
#include <unordered_map>

#include "host_runtime.h"
#include "spec_gate.h"

namespace specv {

struct TenantGate {
  double ema = NAN;
  int32_t state = SPEC_GATE_CLOSED;
  int32_t cooldown = 0;
  int64_t observations = 0;
  int64_t accepted = 0;
  int64_t drafted = 0;
  int64_t trips = 0;
};

}  // namespace specv

struct spec_gate {
  spec_gate_config_t cfg;
  std::mutex lock;
  std::unordered_map<uint64_t, specv::TenantGate> tenants;
};

using namespace specv;

namespace {

void open_breaker(const spec_gate_config_t& cfg, TenantGate& t) {
  t.state = SPEC_GATE_OPEN;
  t.cooldown = cfg.cooldown;
  ++t.trips;
}

void observe_one(const spec_gate_config_t& cfg, TenantGate& t, int32_t acc, int32_t drafted) {
  const double rate = static_cast<double>(acc) / static_cast<double>(drafted);
  ++t.observations;
  t.accepted += acc;
  t.drafted += drafted;
  if (t.state == SPEC_GATE_HALF_OPEN) {
    t.ema = rate;  // recovery is judged afresh
    if (rate >= cfg.acceptance_floor)
      t.state = SPEC_GATE_CLOSED;
    else
      open_breaker(cfg, t);
    return;
  }
  t.ema = std::isnan(t.ema) ? rate : (1.0 - cfg.ema_weight) * t.ema + cfg.ema_weight * rate;
  if (t.state == SPEC_GATE_CLOSED && t.ema < cfg.acceptance_floor) open_breaker(cfg, t);
}

}  // namespace

extern "C" {

void spec_gate_default_config(spec_gate_config_t* cfg) {
  if (!cfg) return;
  cfg->temperature_limit = 0.70;
  cfg->acceptance_floor = 0.55;
  cfg->ema_weight = 0.1;
  cfg->cooldown = 64;
}

spec_status_t spec_gate_create(const spec_gate_config_t* cfg, spec_gate_t** out_gate) {
  if (!out_gate) return fail(SPEC_ERR_INVALID_ARG, "out_gate is NULL");
  *out_gate = nullptr;
  spec_gate_config_t c;
  spec_gate_default_config(&c);
  if (cfg) c = *cfg;
  if (std::isnan(c.temperature_limit)) return fail(SPEC_ERR_INVALID_ARG, "temperature_limit is NaN");
  if (!(c.acceptance_floor >= 0.0 && c.acceptance_floor <= 1.0))
    return fail(SPEC_ERR_INVALID_ARG, "acceptance_floor must lie in [0, 1]");
  if (!(c.ema_weight > 0.0 && c.ema_weight <= 1.0)) return fail(SPEC_ERR_INVALID_ARG, "ema_weight must lie in (0, 1]");
  if (c.cooldown < 1) return fail(SPEC_ERR_INVALID_ARG, "cooldown must be >= 1");
  spec_gate_t* g = new (std::nothrow) spec_gate;
  if (!g) return fail(SPEC_ERR_INVALID_ARG, "out of host memory");
  g->cfg = c;
  *out_gate = g;
  return SPEC_OK;
}

void spec_gate_destroy(spec_gate_t* gate) { delete gate; }

spec_status_t spec_gate_decide(spec_gate_t* gate, const uint64_t* tenant, const float* temperature, int B,
                               int32_t* out_speculate) {
  if (!gate || B < 0) return fail(SPEC_ERR_INVALID_ARG, "need a gate and B >= 0");
  if (B == 0) return SPEC_OK;
  if (!tenant || !temperature || !out_speculate) return fail(SPEC_ERR_INVALID_ARG, "a required pointer is NULL");
  std::lock_guard<std::mutex> hold(gate->lock);
  for (int i = 0; i < B; ++i) {
    TenantGate& t = gate->tenants[tenant[i]];
    const bool t_ok = static_cast<double>(temperature[i]) <= gate->cfg.temperature_limit;  // false for NaN
    out_speculate[i] = t_ok && t.state != SPEC_GATE_OPEN ? 1 : 0;
    if (t.state == SPEC_GATE_OPEN && --t.cooldown == 0) t.state = SPEC_GATE_HALF_OPEN;
  }
  return SPEC_OK;
}

spec_status_t spec_gate_observe(spec_gate_t* gate, const uint64_t* tenant, const int32_t* num_accepted,
                                const int32_t* draft_len, int B) {
  if (!gate || B < 0) return fail(SPEC_ERR_INVALID_ARG, "need a gate and B >= 0");
  if (B == 0) return SPEC_OK;
  if (!tenant || !num_accepted || !draft_len) return fail(SPEC_ERR_INVALID_ARG, "a required pointer is NULL");
  std::lock_guard<std::mutex> hold(gate->lock);
  for (int i = 0; i < B; ++i) {
    const int32_t a = num_accepted[i], d = draft_len[i];
    if (d <= 0 || a < 0 || a > d) continue;
    observe_one(gate->cfg, gate->tenants[tenant[i]], a, d);
  }
  return SPEC_OK;
}

spec_status_t spec_gate_tenant(spec_gate_t* gate, uint64_t tenant, spec_gate_tenant_stats_t* out) {
  if (!gate || !out) return fail(SPEC_ERR_INVALID_ARG, "need a gate and an output");
  std::lock_guard<std::mutex> hold(gate->lock);
  const auto it = gate->tenants.find(tenant);
  const TenantGate t = it == gate->tenants.end() ? TenantGate{} : it->second;
  out->ema = t.ema;
  out->state = t.state;
  out->cooldown = t.cooldown;
  out->observations = t.observations;
  out->accepted = t.accepted;
  out->drafted = t.drafted;
  out->trips = t.trips;
  return SPEC_OK;
}

int64_t spec_gate_tenant_count(spec_gate_t* gate) {
  if (!gate) return -1;
  std::lock_guard<std::mutex> hold(gate->lock);
  return static_cast<int64_t>(gate->tenants.size());
}

}  // extern "C"
