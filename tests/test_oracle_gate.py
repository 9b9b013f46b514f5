"""Pins of the adaptive-gate oracle (CPU only).

The page fixes the temperature limit (0.70, "above" suppresses), the acceptance floor
(0.55, "below" trips) and that the rolling rate is an exponential moving average per
tenant.  Pins: the thresholds at and around their values, the EMA's closed form
ema_k = b + (a - b)(1 - w)^k for a stream a, b, b, ..., the trip step predicted from
that closed form with logarithms, tenant isolation, the cooldown count and both trial
outcomes, and planted mistakes that must each fail one of them.
"""

import math

import pytest

import oracle.gate as og


def test_temperature_limit_boundary():
    g = og.Gate()
    assert g.decide(1, 0.70) is True
    assert g.decide(1, 0.0) is True
    assert g.decide(1, math.nextafter(0.70, 1.0)) is False
    assert g.decide(1, 1.5) is False
    assert g.decide(1, math.nan) is False


def test_floor_boundary_and_first_observation():
    g = og.Gate()
    g.observe(7, 11, 20)   # 0.55 exactly: not below the floor
    assert g.tenants[7].ema == 0.55 and g.tenants[7].state == og.CLOSED
    g2 = og.Gate()
    g2.observe(7, 10, 20)  # 0.5 < 0.55 trips at once
    assert g2.tenants[7].state == og.OPEN and g2.tenants[7].trips == 1
    assert g2.decide(7, 0.1) is False


@pytest.mark.parametrize("a,b,w", [(1.0, 0.2, 0.1), (0.8, 0.4, 0.25), (0.9, 0.0, 0.05), (0.6, 0.5, 0.3)])
def test_ema_closed_form_and_trip_step(a, b, w):
    g = og.Gate(ema_weight=w)
    g.observe(3, round(a * 20), 20)
    k_trip = math.ceil(math.log((0.55 - b) / (a - b)) / math.log(1.0 - w))
    for k in range(1, k_trip + 1):
        assert g.tenants[3].state == og.CLOSED
        g.observe(3, round(b * 20), 20)
        assert g.tenants[3].ema == pytest.approx(b + (a - b) * (1 - w) ** k, rel=1e-12, abs=1e-15)
    assert g.tenants[3].state == og.OPEN
    assert g.tenants[3].trips == 1


def test_constant_stream_keeps_its_rate():
    g = og.Gate(ema_weight=0.2)
    for _ in range(50):
        g.observe(5, 3, 4)
    assert g.tenants[5].ema == pytest.approx(0.75, rel=1e-14)
    assert g.tenants[5].observations == 50 and g.tenants[5].accepted == 150 and g.tenants[5].drafted == 200


def test_invalid_steps_are_not_observations():
    g = og.Gate()
    for acc, dr in ((0, 0), (-1, 5), (6, 5), (2, -3)):
        g.observe(9, acc, dr)
    assert 9 not in g.tenants or g.tenants[9].observations == 0


def test_tenants_are_isolated():
    g = og.Gate()
    g.observe(1, 0, 5)
    g.observe(2, 5, 5)
    assert g.decide(1, 0.5) is False and g.decide(2, 0.5) is True and g.decide(3, 0.5) is True


def test_cooldown_then_trial_outcomes():
    C = 5
    g = og.Gate(cooldown=C)
    g.observe(4, 0, 5)
    decisions = [g.decide(4, 0.2) for _ in range(C)]
    assert decisions == [False] * C
    assert g.tenants[4].state == og.HALF_OPEN
    assert g.decide(4, 0.2) is True and g.decide(4, 0.9) is False  # the T gate still applies
    g.observe(4, 1, 5)  # trial fails: reopen with a fresh cooldown
    assert g.tenants[4].state == og.OPEN and g.tenants[4].ema == 0.2 and g.tenants[4].trips == 2
    assert [g.decide(4, 0.2) for _ in range(C)] == [False] * C
    g.observe(4, 3, 5)  # trial succeeds: the EMA restarts at 0.6
    assert g.tenants[4].state == og.CLOSED and g.tenants[4].ema == 0.6
    assert g.decide(4, 0.2) is True


# ------------------------------------------------------------ planted mistakes
class NonStrictFloor(og.Gate):
    def observe(self, key, accepted, drafted):
        super().observe(key, accepted, drafted)
        t = self.tenants.get(key)
        if t and t.state == og.CLOSED and t.ema <= self.floor:
            t.state, t.cooldown = og.OPEN, self.cooldown


class SwappedWeight(og.Gate):
    def __init__(self, **kw):
        super().__init__(**kw)
        self.w = 1.0 - self.w


class InclusiveTemperature(og.Gate):
    def decide(self, key, temperature):
        r = super().decide(key, temperature)
        return r and temperature < self.limit


class ShortCooldown(og.Gate):
    def __init__(self, **kw):
        super().__init__(**kw)
        self.cooldown -= 1


@pytest.mark.parametrize("cls", [NonStrictFloor, SwappedWeight, InclusiveTemperature, ShortCooldown])
def test_planted_mistakes_are_caught(monkeypatch, cls):
    monkeypatch.setattr(og, "Gate", cls)
    pins = [test_temperature_limit_boundary, test_floor_boundary_and_first_observation,
            lambda: test_ema_closed_form_and_trip_step(1.0, 0.2, 0.1), test_cooldown_then_trial_outcomes]
    failed = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1
