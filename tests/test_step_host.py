"""IndexerStep's pinned staging ring (host logic, CPU): a staging buffer is
rewritten only after the host has waited on an event recorded at or after
the upload that last read it, and events are recorded on one plan in
GUARD_EVERY, not on every one."""

import collections

import pytest

import sparse_attention_block_mxfp4_amd.step as step_mod


class _Log:
    def __init__(self):
        self.plans = 0            # plans enqueued so far
        self.waited = -1          # highest plan number covered by a waited event
        self.events = 0
        self.writes = []          # (plan number, buffer, covered plan number at the time)


def _fake_step(log, monkeypatch):
    class FakeEvent:
        def record(self, stream=None):
            self.covers = log.plans - 1       # every upload enqueued before it
            log.events += 1

        def synchronize(self):
            log.waited = max(log.waited, self.covers)

    class FakeCuda:
        Event = FakeEvent

        @staticmethod
        def current_stream():
            return None

    class FakeTorch:
        cuda = FakeCuda

    def fake_plan(cu, sl, H, budget, staging, plan, stream=None):
        log.writes.append((log.plans, staging, log.waited))
        log.plans += 1
        return object()

    monkeypatch.setattr(step_mod, "torch", FakeTorch)
    monkeypatch.setattr(step_mod, "mi_idx_plan_prefill", fake_plan)
    s = object.__new__(step_mod.IndexerStep)
    s.H, s.query_len, s.max_pages = 4, 1, 64
    s.dec_plan = s.dec_ws = None
    s.pre_plan = "plan"
    s.pre_staging = [f"buf{i}" for i in range(step_mod.NSTAGE)]
    s._plans = 0
    s._guards = collections.deque()
    s.pre_launch = None
    return s


@pytest.mark.parametrize("steps", [1, 15, 16, 17, 100])
def test_staging_ring_waits_before_reuse(monkeypatch, steps):
    log = _Log()
    s = _fake_step(log, monkeypatch)
    for _ in range(steps):
        s.plan(None, [0, 4], [10], gather_budget_pages=0)
    assert len(log.writes) == steps
    last_use = {}
    for n, buf, waited in log.writes:
        assert buf == f"buf{n % step_mod.NSTAGE}"
        if buf in last_use:
            # the upload of the plan that last used this buffer is complete
            assert waited >= last_use[buf], (n, buf, waited, last_use[buf])
        last_use[buf] = n
    assert log.events == -(-steps // step_mod.GUARD_EVERY)
    assert step_mod.GUARD_EVERY < step_mod.NSTAGE
