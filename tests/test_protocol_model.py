"""A CPU model of the exchange protocol of the persistent batch-1 stack kernel (k_flow2), run under
many random interleavings.

What the model keeps from the kernel:
  - one global iteration counter it = t * L + l per (token, layer); every word a workgroup
    publishes in iteration it carries the epoch it + 1;
  - per-layer word slots: h[l] (role 2 -> role 1, read one iteration later), g[l] (role 1 -> role 2),
    bc[l] (role 1 -> the role-1 items of the same group), and the fold factor rx (role-1 workgroup 0
    -> every role-2 workgroup at layer 0 of every token after the first);
  - the slots start cleared (epoch 0) and the last layer's h slot is seeded with x0 at epoch 0;
  - a reader polls its words (one word per load here: no two words are assumed to arrive
    together) until every epoch equals the one it wants, with a bounded number of polls; past the
    bound it raises the shared error flag, and every wait that sees the flag gives up at once;
  - after the kernel, the finish step reports the flag and fills y with NaN when it is set.
The payload arithmetic is replaced by exact integer functions with the same data dependences
(every h word feeds every role-1 item, every g word every role-2 row, the group's B/C words every
item of the group), so a sequential evaluation gives the reference values.

Checked: for random schedules every output equals the sequential reference, no word is ever
overwritten while a reader that needs it has not read it (the reuse rule of the per-layer
slots), no reader ever sees an epoch newer than the one it waits for, the error flag stays clear;
with a producer that stops, every workgroup still ends within the poll bound, the flag is set and
y is NaN. Negative controls (a reader that does not check epochs, a role-2 workgroup that skips the
fold wait) must be caught.
"""
import random

import numpy as np
import pytest

MOD = 1_000_003


class Violation(Exception):
    pass


class Memory:
    """Tagged words {payload, epoch}; tracks, for every word, the readers that still need its current
    epoch, so that a store over a word someone has yet to read is a protocol violation."""

    def __init__(self):
        self.words = {}
        self.pending = {}
        self.err = 0

    def store(self, key, payload, epoch, readers):
        # once the flag is up the data is void anyway (readers gave up without reading)
        if self.pending.get(key) and not self.err:
            raise Violation(f"{key} overwritten at epoch {epoch} before {sorted(self.pending[key])} read it")
        self.words[key] = (payload, epoch)
        self.pending[key] = set(readers)

    def load(self, key):
        return self.words.get(key, (0, 0))

    def consumed(self, key, reader):
        self.pending.get(key, set()).discard(reader)


class Cfg:
    def __init__(self, L=3, T=4, G=2, per_group=2, n2=3, rows_per_r2=2, spin=400):
        self.L, self.T, self.G, self.per_group, self.n2, self.rows_per_r2, self.spin = L, T, G, per_group, n2, rows_per_r2, spin
        self.n1 = G * per_group
        self.D = n2 * rows_per_r2        # h words (role-2 workgroup j owns rows j*R .. j*R+R-1)
        self.E = self.n1                 # g words (one per role-1 item)


def f_bc(H, l, i):
    return (H + 7 * i + 3 * l) % MOD


def f_g(H, BC, l, i):
    return (3 * H + BC + 11 * i + l) % MOD


def f_h(h_old, Gs, l, r):
    return (h_old + Gs + 5 * r + 2 * l) % MOD


def f_fold(H):
    return H % 97 + 1


def reference(cfg, x0):
    h = list(x0)
    ys = []
    for t in range(cfg.T):
        if t > 0:
            r = f_fold(sum(h) % MOD)
            h = [v * r % MOD for v in h]
            ys.append(list(h))
        for l in range(cfg.L):
            H = sum(h) % MOD
            bc = [f_bc(H, l, i) for i in range(cfg.n1)]
            g = []
            for i in range(cfg.n1):
                grp = i // cfg.per_group
                BC = sum(bc[grp * cfg.per_group:(grp + 1) * cfg.per_group]) % MOD
                g.append(f_g(H, BC, l, i))
            Gs = sum(g) % MOD
            h = [f_h(h[r], Gs, l, r) for r in range(cfg.D)]
    r = f_fold(sum(h) % MOD)
    ys.append([v * r % MOD for v in h])
    return ys


def gather(mem, cfg, keys, epoch, me, check_epochs=True):
    """Poll `keys` until every epoch equals `epoch` (bounded). Returns payloads, or None on timeout
    or when the error flag is up."""
    spins = 0
    while True:
        vals, ok = [], True
        for k in keys:
            p, e = mem.load(k)
            yield
            if e > epoch and check_epochs and not mem.err:
                raise Violation(f"{me} waiting for epoch {epoch} of {k} saw {e}")
            if e != epoch and check_epochs:
                ok = False
            vals.append(p)
        if ok:
            for k in keys:
                mem.consumed(k, me)
            return vals
        spins += 1
        if mem.err:
            return None
        if spins > cfg.spin:
            mem.err = 1
            return None
        yield


def role1(mem, cfg, i, out, faults):
    me = ("r1", i)
    grp = i // cfg.per_group
    L = cfg.L
    for t in range(cfg.T):
        for l in range(L):
            it = t * L + l
            tag = it + 1
            lp = L - 1 if l == 0 else l - 1
            hv = yield from gather(mem, cfg, [("h", lp, r) for r in range(cfg.D)], tag - 1, me,
                                   check_epochs=not faults.get("no_epoch_check"))
            if hv is None:
                hv = [0] * cfg.D
            if l == 0 and t > 0:
                r0 = f_fold(sum(hv) % MOD)
                hv = [v * r0 % MOD for v in hv]
                if i == 0:
                    out["y"][t - 1] = list(hv)
                    mem.store(("rx",), r0, tag, readers=[("r2", j) for j in range(cfg.n2)])
                    yield
            H = sum(hv) % MOD
            if faults.get("dead") == (i, it):
                return   # this producer stops: its words never appear
            mem.store(("bc", l, i), f_bc(H, l, i), tag,
                      readers=[("r1", k) for k in range(grp * cfg.per_group, (grp + 1) * cfg.per_group)])
            yield
            bc = yield from gather(mem, cfg, [("bc", l, k) for k in range(grp * cfg.per_group, (grp + 1) * cfg.per_group)],
                                   tag, me)
            BC = sum(bc) % MOD if bc is not None else 0
            mem.store(("g", l, i), f_g(H, BC, l, i), tag, readers=[("r2", j) for j in range(cfg.n2)])
            yield
    if i == 0:
        hv = yield from gather(mem, cfg, [("h", L - 1, r) for r in range(cfg.D)], cfg.T * L, me)
        if hv is None:
            hv = [0] * cfg.D
        r0 = f_fold(sum(hv) % MOD)
        out["y"][cfg.T - 1] = [v * r0 % MOD for v in hv]


def role2(mem, cfg, j, x0, faults):
    me = ("r2", j)
    rows = list(range(j * cfg.rows_per_r2, (j + 1) * cfg.rows_per_r2))
    hold = [x0[r] for r in rows]
    L = cfg.L
    for t in range(cfg.T):
        for l in range(L):
            it = t * L + l
            tag = it + 1
            if l == 0 and t > 0:
                if faults.get("skip_fold_wait"):
                    r0, _ = mem.load(("rx",))
                    yield
                else:
                    v = yield from gather(mem, cfg, [("rx",)], tag, me)
                    r0 = v[0] if v is not None else 0
                hold = [h * r0 % MOD for h in hold]
            gv = yield from gather(mem, cfg, [("g", l, k) for k in range(cfg.n1)], tag, me)
            Gs = sum(gv) % MOD if gv is not None else 0
            hold = [f_h(hold[k], Gs, l, r) for k, r in enumerate(rows)]
            for k, r in enumerate(rows):
                last = it + 1 == cfg.T * L   # read only by the final norm of role-1 workgroup 0
                mem.store(("h", l, r), hold[k], tag,
                          readers=[("r1", 0)] if last else [("r1", i) for i in range(cfg.n1)])
                yield


def run(cfg, seed, faults=None):
    faults = faults or {}
    rng = random.Random(seed)
    mem = Memory()
    x0 = [rng.randrange(MOD) for _ in range(cfg.D)]
    for r in range(cfg.D):   # k_seed2: x0 into the last layer's h slot at epoch 0
        mem.store(("h", cfg.L - 1, r), x0[r], 0, readers=[("r1", i) for i in range(cfg.n1)])
    out = {"y": [None] * cfg.T}
    procs = [role1(mem, cfg, i, out, faults) for i in range(cfg.n1)] + \
            [role2(mem, cfg, j, x0, faults) for j in range(cfg.n2)]
    live = list(range(len(procs)))
    steps = 0
    while live:
        k = rng.choice(live)
        try:
            next(procs[k])
        except StopIteration:
            live.remove(k)
        steps += 1
        assert steps < 5_000_000, "model did not terminate"
    # the finish step: report the flag, NaN-fill y when it is set
    y = np.array([[np.nan] * cfg.D if (mem.err or v is None) else v for v in out["y"]], dtype=float)
    return mem.err, y, reference(cfg, x0)


@pytest.mark.parametrize("seed", range(40))
def test_random_schedules_match_the_sequential_reference(seed):
    cfg = Cfg(L=2 + seed % 3, T=2 + seed % 4, G=1 + seed % 2, per_group=1 + seed % 3, n2=1 + seed % 3,
              rows_per_r2=1 + (seed // 3) % 2, spin=10_000)
    err, y, ref = run(cfg, seed)
    assert err == 0
    assert np.array_equal(y, np.array(ref, dtype=float))


@pytest.mark.parametrize("seed", range(10))
def test_a_dead_producer_ends_every_workgroup_with_the_flag_and_nan(seed):
    cfg = Cfg(L=3, T=3, G=2, per_group=2, n2=2, rows_per_r2=2, spin=200)
    err, y, _ = run(cfg, seed, faults={"dead": (seed % cfg.n1, seed % (cfg.T * cfg.L))})
    assert err == 1
    assert np.isnan(y).all()


def test_negative_control_reader_without_epoch_check_is_caught():
    cfg = Cfg(L=2, T=3, G=1, per_group=2, n2=2, rows_per_r2=1, spin=10_000)
    caught = 0
    for seed in range(30):
        try:
            err, y, ref = run(cfg, seed, faults={"no_epoch_check": True})
            caught += int(not np.array_equal(y, np.array(ref, dtype=float)))
        except Violation:
            caught += 1
    assert caught > 0


def test_negative_control_skipped_fold_wait_is_caught():
    cfg = Cfg(L=2, T=3, G=1, per_group=2, n2=2, rows_per_r2=1, spin=10_000)
    caught = 0
    for seed in range(30):
        try:
            err, y, ref = run(cfg, seed, faults={"skip_fold_wait": True})
            caught += int(not np.array_equal(y, np.array(ref, dtype=float)))
        except Violation:
            caught += 1
    assert caught > 0
