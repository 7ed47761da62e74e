"""Host-side model of the key-split attention schedule (attn_bf16_ks_kernel
in learned_token_pruning_score_amd/csrc/attn.hip).

The model replays, for every wave of a 128-row query tile, the kernel's
sequence of staging loads and stores, score and value products, softmaxes
and barriers, in the order the kernel issues them, and checks what a wrong
schedule would break on the GPU: every wave passes the same number of
barriers (else the workgroup hangs), every LDS stage is written before it
is read and not overwritten in between, each staging store writes the tile
its registers were loaded with, and every key tile of every active row is
scored, normalised and multiplied exactly once, by the group that owns it.
A change to the kernel's schedule must be mirrored here.
"""
import itertools

kBK, BQ = 64, 128

def run(n, q0):
    kv_end = min(q0 + BQ, n); n_kt = (kv_end + kBK - 1) // kBK; n_int = n_kt + 3
    waves = []
    for wave in range(8):
        grp, pair = wave >> 2, wave & 3
        qw = q0 + 32 * pair
        active = qw < n
        t_diag = min(qw + 31, n - 1) // kBK if active else -1
        ev = []  # list of (interval, op, tile)
        st = {'i': -1, 'hreg': None}
        def barrier(): st['i'] += 1; ev.append((st['i'], 'bar', None))
        def op(name, t): ev.append((st['i'] + 1, name, t))
        # prologue
        if grp == 0: op('load_k', 0); op('store_k', 0); op('load_v', 0)
        else: op('load_k', 1)
        barrier()  # prologue barrier -> interval index 0 starts after it
        i = 0
        if grp == 1:
            op('store_k', 1); op('load_v', 1); barrier(); i = 1
        if t_diag >= grp:
            t = grp
            op('store_v', t); op('load_k', t + 2); op('qk', t); barrier()
            op('softmax_m' if t == t_diag else 'softmax', t); op('store_k', t + 2); op('load_v', t + 2); barrier()
            t += 2
            while t < t_diag:
                op('store_v', t); op('load_k', t + 2); op('pv', t - 2); op('qk', t); barrier()
                op('softmax', t); op('store_k', t + 2); op('load_v', t + 2); barrier(); t += 2
            if t == t_diag:
                op('store_v', t); op('load_k', t + 2); op('pv', t - 2); op('qk', t); barrier()
                op('softmax_m', t); op('store_k', t + 2); op('load_v', t + 2); barrier(); t += 2
            op('store_v', t); op('load_k', t + 2); op('pv', t - 2); barrier()
            op('store_k', t + 2); op('load_v', t + 2); barrier()
            i = t + 2
        while i < n_int:
            if ((i ^ grp) & 1) == 0: op('store_v', i); op('load_k', i + 2)
            else: op('store_k', i + 1); op('load_v', i + 1)
            barrier(); i += 1
        waves.append(dict(grp=grp, active=active, t_diag=t_diag, ev=ev, qw=qw))
    # 1) barrier counts equal
    nb = [sum(1 for e in w['ev'] if e[1] == 'bar') for w in waves]
    assert len(set(nb)) == 1, (n, q0, nb)
    # interval of an op = number of barriers before it (prologue = -1 -> interval index k means after k+1 barriers)
    # rebuild with interval numbers: ops between barrier j-1 and j belong to "epoch" j (epoch 0 = prologue)
    epochs = []
    for w in waves:
        e, out = 0, []
        for (_, name, t) in w['ev']:
            if name == 'bar': e += 1
            else: out.append((e, name, t))
        epochs.append(out)
    # 2) register hand-off: each store consumes the wave's latest load, same kind and tile
    for w, ops in zip(waves, epochs):
        last = None
        for (e, name, t) in ops:
            if name.startswith('load'): last = (name[5], t)
            elif name.startswith('store'):
                assert last == (name[6], t), (n, q0, w['qw'], w['grp'], e, name, t, last)
                last = None
    # 3) LDS lifetimes: writes by all 4 waves of a group in one epoch; reads later, stage not overwritten between
    writes = {}  # (kind, tile) -> epoch (all writers must agree)
    for w, ops in zip(waves, epochs):
        for (e, name, t) in ops:
            if name.startswith('store'):
                key = (name[6], t)
                writes.setdefault(key, set()).add(e)
    for key, es in writes.items():
        assert len(es) == 1, ('writers disagree', key, es)
    wr = {k: next(iter(v)) for k, v in writes.items()}
    nstage = {'k': 2, 'v': 3}
    for w, ops in zip(waves, epochs):
        for (e, name, t) in ops:
            if name in ('qk', 'pv'):
                kind = 'k' if name == 'qk' else 'v'
                assert (kind, t) in wr, ('never written', n, q0, kind, t)
                we = wr[(kind, t)]
                assert we < e, ('read before write', n, q0, kind, t, we, e)
                # no other tile mapped to the same stage written in epochs (we, e]
                for (k2, t2), e2 in wr.items():
                    if k2 == kind and t2 != t and t2 % nstage[kind] == t % nstage[kind] and we < e2 <= e:
                        raise AssertionError(('overwritten', n, q0, kind, t, t2, we, e2, e))
                # and no write to the same stage in the same epoch as the read (by any group)
    # 4) every needed tile is computed: each active wave's tiles 0..t_diag get qk, softmax and pv exactly once across its pair
    for pair in range(4):
        a, b = waves[pair], waves[pair + 4]
        if not a['active']: continue
        done = {}
        for w, ops in ((a, epochs[pair]), (b, epochs[pair + 4])):
            for (e, name, t) in ops:
                if name in ('qk', 'pv', 'softmax', 'softmax_m'): done.setdefault(t, []).append((name, w['grp']))
        for t in range(a['t_diag'] + 1):
            names = sorted(x[0] for x in done.get(t, []))
            exp = sorted(['qk', 'pv', 'softmax_m' if t == a['t_diag'] else 'softmax'])
            assert names == exp, (n, q0, pair, t, names)
            assert len(set(x[1] for x in done[t])) == 1 and done[t][0][1] == t % 2
        assert all(t <= a['t_diag'] for t in done), (n, q0, pair, sorted(done))
    return nb[0]


def test_key_split_schedule_every_tile():
    count = 0
    for n in list(range(1, 700)) + [1000, 2304, 4352, 8448, 8449, 8511]:
        for q0 in range(0, n, BQ):
            run(n, q0)
            count += 1
    assert count > 2000
