"""Host-side model of the 256-row attention schedule (attn_bf16_kernel in
learned_token_pruning_score_amd/csrc/attn.hip).

The model replays, for every wave of a 256-row query tile, the kernel's
sequence of staging loads and stores, score and value products, softmaxes
and barriers, in the order the kernel issues them, and checks what a wrong
schedule would break on the GPU: every wave passes the same number of
barriers (else the workgroup hangs); every LDS stage half (K rows and bias by
group 0, V rows by group 1) is written before it is read, by one tile only,
and not rewritten until its last read has passed a barrier; each staging
store writes the tile that its register set was loaded with (tile 1 comes
from a register set of its own, loaded with tile 0 in the prologue); and
every key tile of every active row is scored, normalised and multiplied
exactly once, masked only where it crosses the wave's diagonal, and no tile
that a row does not see is used.  A change to the kernel's schedule must be
mirrored here.
"""

kBK, BQ, NSTAGE = 64, 256, 3


def _replay(n, q0, wave):
    grp = wave >> 2
    qw = q0 + 64 * (wave & 3) + 32 * grp
    kv_end = min(q0 + BQ, n)
    n_kt = (kv_end + kBK - 1) // kBK
    n_loop = n_kt + 1
    t_diag = min(qw + 31, n - 1) // kBK if qw < n else -1
    ev = []  # (name, tile, register set); 'bar' separates epochs
    half = 'k' if grp == 0 else 'v'

    def op(name, t, reg=None):
        ev.append((name, t, reg))

    def bar():
        ev.append(('bar', None, None))

    def stage_next(t):  # tile t from the main register set, then load t + 1 into it
        op('store_' + half, t, 'hreg')
        op('load_' + half, t + 1, 'hreg')

    def stage_first():  # tile 1 from its own register set, then load tile 2
        op('store_' + half, 1, 'hreg1')
        op('load_' + half, 2, 'hreg')

    # prologue
    op('load_' + half, 0, 'hreg')
    op('load_' + half, 1, 'hreg1')
    op('store_' + half, 0, 'hreg')
    bar()
    t = 0
    if grp == 0:
        if t_diag >= 0:
            op('qk', 0)
            bar()
            stage_first()
            op('softmax_m' if t_diag == 0 else 'softmax', 0)
            bar()
            t = 1
            while t < t_diag:
                op('pv', t - 1); op('qk', t); bar()
                stage_next(t + 1); op('softmax', t); bar()
                t += 1
            if t == t_diag:
                op('pv', t - 1); op('qk', t); bar()
                stage_next(t + 1); op('softmax_m', t); bar()
                t += 1
            op('pv', t - 1); bar()
            stage_next(t + 1); bar()
            t += 1
        while t < n_loop:
            bar()
            if t == 0:
                stage_first()
            else:
                stage_next(t + 1)
            bar()
            t += 1
    else:
        if t_diag >= 0:
            stage_first(); bar()
            op('qk', 0); bar()
            t = 1
            while t <= t_diag:
                stage_next(t + 1); op('softmax', t - 1); bar()
                op('pv', t - 1); op('qk', t); bar()
                t += 1
            stage_next(t + 1); op('softmax_m', t_diag); bar()
            op('pv', t - 1); bar()
            t += 1
        while t < n_loop:
            if t == 0:
                stage_first()
            else:
                stage_next(t + 1)
            bar(); bar()
            t += 1
    return dict(grp=grp, qw=qw, t_diag=t_diag, active=qw < n, ev=ev)


def run(n, q0):
    waves = [_replay(n, q0, w) for w in range(8)]
    # 1) every wave passes the same number of barriers
    nb = [sum(1 for e in w['ev'] if e[0] == 'bar') for w in waves]
    assert len(set(nb)) == 1, (n, q0, nb)
    # epochs: ops between barrier j - 1 and j belong to epoch j (epoch 0 = before the first barrier)
    epochs = []
    for w in waves:
        e, out = 0, []
        for (name, t, reg) in w['ev']:
            if name == 'bar':
                e += 1
            else:
                out.append((e, name, t, reg))
        epochs.append(out)
    # 2) register hand-off: a store writes what its register set was last loaded with
    for w, ops in zip(waves, epochs):
        held = {}
        for (e, name, t, reg) in ops:
            if name.startswith('load'):
                held[reg] = t
            elif name.startswith('store'):
                assert held.get(reg) == t, (n, q0, w['qw'], e, name, t, reg, held)
                held[reg] = None  # consumed
    # 3) LDS: the writes of a stage half in one epoch are of one tile, by all 4 waves of its group;
    # reads come later and the half is not rewritten before (or in) the epoch of the read
    writes = {}  # (half, stage) -> list of (epoch, tile)
    for ops in epochs:
        for (e, name, t, reg) in ops:
            if name.startswith('store'):
                writes.setdefault((name[6], t % NSTAGE), set()).add((e, t))
    for key, ws in writes.items():
        by_epoch = {}
        for (e, t) in ws:
            by_epoch.setdefault(e, set()).add(t)
        assert all(len(ts) == 1 for ts in by_epoch.values()), ('two tiles in one epoch', n, q0, key, by_epoch)
    for w, ops in zip(waves, epochs):
        for (e, name, t, reg) in ops:
            if name not in ('qk', 'pv'):
                continue
            h = 'k' if name == 'qk' else 'v'
            ws = sorted(writes.get((h, t % NSTAGE), ()))
            before = [(we, wt) for (we, wt) in ws if we < e]
            assert before and before[-1][1] == t, ('stage holds another tile', n, q0, w['qw'], name, t, e, ws)
            assert not any(we == e for (we, wt) in ws), ('write in the epoch of a read', n, q0, name, t, e, ws)
    # 4) each active wave runs qk, softmax (masked on its diagonal tile only) and pv of tiles
    # 0 .. t_diag exactly once, in that order, and a tile before the diagonal is visible to all its rows
    for w, ops in zip(waves, epochs):
        done = {}
        for (e, name, t, reg) in ops:
            if name in ('qk', 'softmax', 'softmax_m', 'pv'):
                done.setdefault(t, []).append((e, name))
        if not w['active']:
            assert not done, (n, q0, w['qw'], done)
            continue
        assert sorted(done) == list(range(w['t_diag'] + 1)), (n, q0, w['qw'], sorted(done))
        for t, lst in done.items():
            names = [x[1] for x in sorted(lst)]
            sm = 'softmax_m' if t == w['t_diag'] else 'softmax'
            assert names == ['qk', sm, 'pv'], (n, q0, w['qw'], t, names)
            if t < w['t_diag']:
                assert kBK * t + kBK - 1 <= w['qw'], (n, q0, w['qw'], t)  # no key past the wave's first row
    return nb[0]


def test_tile_schedule_every_tile():
    count = 0
    for n in list(range(1, 1100)) + [2304, 4352, 8448, 8449, 8511, 16640]:
        for q0 in range(0, n, BQ):
            run(n, q0)
            count += 1
    assert count > 2000

