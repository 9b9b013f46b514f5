"""Acceptance telemetry and the adaptive speculation gate -- oracle (TEST INFRASTRUCTURE ONLY).

Page: "Breaking the Memory Bandwidth Wall: 3.42x Generation Speedup with EAGLE Speculative
Decoding" (acefleet.dev), "Closed-Loop Real-Time Adaptive Gating":
  1. a request whose sampling temperature is above 0.70 is served without speculation;
  2. an exponential moving average of the draft acceptance rate is kept per tenant key;
     when it drops below 0.55 a circuit breaker trips and the tenant is served without
     speculation until its predictability recovers.

Readings taken where the page is silent:
  * One observation is one verification step of one sequence: rate = accepted / drafted.
    A step with drafted <= 0, accepted < 0 or accepted > drafted (an invalid sequence)
    is not an observation.
  * EMA: the first observation of a tenant sets it to the rate; later ones move it by
    ema <- (1 - w) * ema + w * rate (w = ema_weight, default 0.1).  Observations of one
    batch apply in batch order.
  * Breaker states per tenant: closed (speculate), open (do not), half-open (speculate on
    trial).  Closed -> open when, after an observation, ema < floor (strictly below).
    While open, every gate decision for the tenant is a refusal and counts down the
    cooldown (default 64 decisions); when it reaches 0 the tenant is half-open.  The first
    observation in half-open restarts the EMA at that rate (recovery is judged afresh)
    and closes the breaker if it is >= floor, else reopens it with a new cooldown.
  * A decision speculates iff temperature <= limit (not NaN) and the tenant's breaker is
    not open.  A tenant never seen is closed.
  * Telemetry per tenant: observations, accepted and drafted totals, trips.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

CLOSED, OPEN, HALF_OPEN = 0, 1, 2


@dataclass
class TenantState:
    state: int = CLOSED
    ema: float = math.nan  # undefined until the first observation
    cooldown: int = 0
    observations: int = 0
    accepted: int = 0
    drafted: int = 0
    trips: int = 0


class Gate:
    def __init__(self, temperature_limit=0.70, acceptance_floor=0.55, ema_weight=0.1, cooldown=64):
        self.limit = float(temperature_limit)
        self.floor = float(acceptance_floor)
        self.w = float(ema_weight)
        self.cooldown = int(cooldown)
        self.tenants = {}

    def _get(self, key):
        if key not in self.tenants:
            self.tenants[key] = TenantState()
        return self.tenants[key]

    def decide(self, key, temperature):
        t = self._get(key)
        allowed_t = temperature <= self.limit  # False for NaN
        speculate = allowed_t and t.state != OPEN
        if t.state == OPEN:
            t.cooldown -= 1
            if t.cooldown == 0:
                t.state = HALF_OPEN
        return speculate

    def observe(self, key, accepted, drafted):
        accepted, drafted = int(accepted), int(drafted)
        if drafted <= 0 or accepted < 0 or accepted > drafted:
            return
        t = self._get(key)
        rate = accepted / drafted
        t.observations += 1
        t.accepted += accepted
        t.drafted += drafted
        if t.state == HALF_OPEN:
            t.ema = rate
            if rate >= self.floor:
                t.state = CLOSED
            else:
                t.state = OPEN
                t.cooldown = self.cooldown
                t.trips += 1
            return
        t.ema = rate if math.isnan(t.ema) else (1.0 - self.w) * t.ema + self.w * rate
        if t.state == CLOSED and t.ema < self.floor:
            t.state = OPEN
            t.cooldown = self.cooldown
            t.trips += 1

    def decide_batch(self, keys, temperatures):
        return [self.decide(int(k), float(T)) for k, T in zip(keys, temperatures)]

    def observe_batch(self, keys, accepted, drafted):
        for k, a, d in zip(keys, accepted, drafted):
            self.observe(int(k), a, d)
