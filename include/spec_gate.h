/*
 * spec_gate.h -- acceptance telemetry and the adaptive speculation gate of
 * libspecverify.so (host-side: plain host memory, no GPU work, no streams).
 *
 * "Breaking the Memory Bandwidth Wall: 3.42x Generation Speedup with EAGLE
 * Speculative Decoding" (acefleet.dev), "Closed-Loop Real-Time Adaptive Gating":
 * a request whose sampling temperature is above 0.70 is served without
 * speculation, and a per-tenant exponential moving average of the draft
 * acceptance rate trips a circuit breaker when it drops below 0.55, serving the
 * tenant without speculation until its predictability recovers.
 *
 * Readings where the page is silent:
 *   - One observation = one verification step of one sequence, rate =
 *     accepted / drafted; steps with drafted <= 0, accepted < 0 or
 *     accepted > drafted are not observations.  A batch applies in index order.
 *   - EMA: the first observation sets it to the rate; later ones apply
 *     ema <- (1 - w) * ema + w * rate, in double precision.
 *   - Breaker per tenant: closed -> open when ema < floor after an observation.
 *     While open every decision for the tenant is a refusal and counts the
 *     cooldown down; at 0 the tenant is half-open.  The first observation in
 *     half-open restarts the EMA at its rate, closing the breaker if that is
 *     >= floor and reopening it (fresh cooldown) otherwise.
 *   - A decision speculates iff temperature <= limit (NaN never does) and the
 *     tenant's breaker is not open.  Unknown tenants are closed.
 *
 * Thread safety: every call on one gate takes the gate's lock.  Tenant state
 * grows with the number of distinct keys and lives until spec_gate_destroy.
 */
#ifndef SPEC_GATE_H
#define SPEC_GATE_H

#include <stddef.h>
#include <stdint.h>

#include "spec_verify.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct spec_gate spec_gate_t; /* opaque */

typedef struct spec_gate_config {
  double temperature_limit; /* speculate only at T <= limit; the page's 0.70 */
  double acceptance_floor;  /* trip when the EMA is below this; the page's 0.55, in [0, 1] */
  double ema_weight;        /* w in (0, 1]; default 0.1 */
  int32_t cooldown;         /* refused decisions before a trial, >= 1; default 64 */
} spec_gate_config_t;

#define SPEC_GATE_CLOSED 0
#define SPEC_GATE_OPEN 1
#define SPEC_GATE_HALF_OPEN 2

typedef struct spec_gate_tenant_stats {
  double ema;            /* NaN before the first observation */
  int32_t state;         /* SPEC_GATE_* */
  int32_t cooldown;      /* refusals left while open */
  int64_t observations;
  int64_t accepted;      /* sum of accepted drafts over the observations */
  int64_t drafted;       /* sum of drafted tokens over the observations */
  int64_t trips;         /* times the breaker opened */
} spec_gate_tenant_stats_t;

/* Fills *cfg with the defaults (0.70, 0.55, 0.1, 64). */
void spec_gate_default_config(spec_gate_config_t* cfg);

/* Creates a gate (host allocation).  cfg NULL = defaults.  INVALID_ARG for a
 * NaN limit, a floor outside [0, 1], a weight outside (0, 1] or cooldown < 1. */
spec_status_t spec_gate_create(const spec_gate_config_t* cfg, spec_gate_t** out_gate);

void spec_gate_destroy(spec_gate_t* gate);

/* For each of B requests (HOST arrays): out_speculate[i] = 1 to speculate, 0 to
 * serve without.  tenant [B], temperature [B] (float). */
spec_status_t spec_gate_decide(spec_gate_t* gate, const uint64_t* tenant, const float* temperature, int B,
                               int32_t* out_speculate);

/* Feeds B verification outcomes (HOST arrays): tenant [B], num_accepted [B] and
 * draft_len [B] (e.g. spec_verify_chain's num_accepted and the draft lengths,
 * copied to the host). */
spec_status_t spec_gate_observe(spec_gate_t* gate, const uint64_t* tenant, const int32_t* num_accepted,
                                const int32_t* draft_len, int B);

/* Telemetry of one tenant (a tenant never seen reads as closed with no data). */
spec_status_t spec_gate_tenant(spec_gate_t* gate, uint64_t tenant, spec_gate_tenant_stats_t* out);

/* Number of tenants the gate holds state for. */
int64_t spec_gate_tenant_count(spec_gate_t* gate);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_GATE_H */
