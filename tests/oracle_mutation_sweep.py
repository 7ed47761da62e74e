"""Mutation sweep of the oracle (test infrastructure, CPU only; run by hand:
``python tests/oracle_mutation_sweep.py``).

Each entry below changes one step of ``oracle/tokengate.py`` the way a
plausible mistake would (a dropped term, a wrong sign, index or operand, an
off-by-one, a wrong reduction).  The sweep applies each to a copy of the
oracle in a temporary directory, runs the CPU pins
(``tests/test_oracle_pins.py``) against it, and reports every mutation the
pins fail to catch.  Exit status 1 if any survives.
"""
import os, shutil, subprocess, sys, tempfile
R = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MUTS = [
 # plan
 ("kept = min(bud[b], doc) + (n - doc)", "kept = min(bud[b], doc) + n"),
 ("kept = min(bud[b], doc) + (n - doc)", "kept = max(bud[b], doc) + (n - doc)"),
 ("longest = max(longest, int(kept))", "longest = max(longest, int(n))"),
 # gate
 ("z = a / (1.0 + np.exp(-a))\n            out", "z = 1.0 / (1.0 + np.exp(-a))\n            out"),
 ("a = h[lo:lo + 8192] @ W.T + bias1[None, :]", "a = h[lo:lo + 8192] @ W.T - bias1[None, :]"),
 ("out[lo:lo + 8192] = z @ w + float(b2)", "out[lo:lo + 8192] = z @ w"),
 ("out[lo:lo + 8192] = z @ w + float(b2)", "out[lo:lo + 8192] = a @ w + float(b2)"),
 # select
 ("order = np.lexsort((idx, -v))", "order = np.lexsort((-idx, -v))"),
 ("order = np.lexsort((idx, -v))", "order = np.lexsort((idx, v))"),
 ("        keep[dlo:dhi] = 0\n", ""),
 ("k = int(min(bud[b], dhi - dlo))", "k = int(min(bud[b], dhi - dlo)) - 1"),
 ("v = s[dlo:dhi].astype(np.float64) + 0.0", "v = np.nan_to_num(s[dlo:dhi].astype(np.float64), nan=np.inf) + 0.0"),
 # compact
 ("bias = np.where(in_doc[kept_idx], sc, np.float32(0.0)).astype(np.float32)", "bias = sc.astype(np.float32)"),
 ("pos_k = np.asarray(pos, dtype=np.int32)[kept_idx]", "pos_k = kept_idx.astype(np.int32)"),
 ("in_doc[cu[b] + db[b]:cu[b] + de[b]] = True", "in_doc[cu[b] + db[b]:cu[b] + de[b] + 1] = True"),
 # attention
 ("                x = scale * (Q[rr, h, :] @ K[lo:lo + n_keys, kv, :].T)", "                x = (Q[rr, h, :] @ K[lo:lo + n_keys, kv, :].T) / math.sqrt(d)"),
 ("                    x = x + g[h] * s[lo:lo + n_keys][None, :]", "                    x = x + s[lo:lo + n_keys][None, :]"),
 ("visible = np.arange(n_keys)[None, :] <= i_rel[:, None]", "visible = np.arange(n_keys)[None, :] < i_rel[:, None] + (i_rel[:, None] == 0)"),
 ("                kv = h // group\n                x = scale", "                kv = h % K.shape[1]\n                x = scale"),
 ("                lse[h, rr] = m + np.log(z)", "                lse[h, rr] = np.log(z)"),
 ("scale = float(tau) / math.sqrt(d)\n    for b in range(cu.shape[0] - 1):\n        lo, hi = int(cu[b]), int(cu[b + 1])\n        if hi == lo:\n            continue\n        if want", "scale = float(tau) / d\n    for b in range(cu.shape[0] - 1):\n        lo, hi = int(cu[b]), int(cu[b + 1])\n        if hi == lo:\n            continue\n        if want"),
 # rope / layer
 ("return np.power(float(theta), -2.0 * i / d)", "return np.power(float(theta), -1.0 * i / d)"),
 ("return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)", "return np.concatenate([a * c + b * s, b * c - a * s], axis=-1)"),
 ("    return apply_rope(q, pos, theta), apply_rope(k, pos, theta), v", "    return apply_rope(q, pos, theta), k, v"),
 ("    return _f64(weight) * x / np.sqrt(ms + float(eps))", "    return _f64(weight) * x / np.sqrt(ms)"),
 ("    return _f64(weight) * x / np.sqrt(ms + float(eps))", "    return x / np.sqrt(ms + float(eps))"),
 ("    return g / (1.0 + np.exp(-g)) * u", "    return u / (1.0 + np.exp(-u)) * g"),
 ("    return linear_residual(swiglu(rms_norm(a, w_post, eps), W_gate, W_up), W_down, a)", "    return linear_residual(swiglu(rms_norm(a, w_in, eps), W_gate, W_up), W_down, a)"),
 ("    a = linear_residual(o[sel].reshape(len(sel), Hq * d), W_o, x[sel])", "    a = linear_residual(o[sel].reshape(len(sel), Hq * d), W_o, 0 * x[sel])"),
 # backward
 ("            dx = P * (dP - np.sum(dOh * O, axis=1, keepdims=True))", "            dx = P * dP"),
 ("            dk[lo:hi, kv] += scale * (dx.T @ Qh)", "            dk[lo:hi, kv] = scale * (dx.T @ Qh)"),
 ("            dv[lo:hi, kv] += P.T @ dOh", "            dv[lo:hi, kv] += P @ dOh"),
 ("                ds[lo:hi] += g[h] * col", "                ds[lo:hi] += col"),
 ("            dtau += float(np.sum(dx * qk)) / math.sqrt(d)", "            dtau += float(np.sum(dx * qk)) / d"),
 ("                dg[h] += float(col @ sb)", "                dg[h] += float(col.sum())"),
 ("            dx = P * (dOi @ V[j, kv] - D)", "            dx = P * (dOi @ V[j, kv])"),
 ("            P = np.exp(x - L[h, j:hi])", "            P = np.exp(x - L[h, j:hi].max())"),
 ("            dx = P * (dP - dO[i, h] @ (P @ Vh))", "            dx = P * dP"),
 # gate backward, score grad
 ("    da = g[:, None] * w[None, :] * sig * (1.0 + a * (1.0 - sig))", "    da = g[:, None] * w[None, :] * sig"),
 ("    return da @ W, da.T @ H, da.sum(axis=0), z.T @ g, float(g.sum())", "    return da @ W, da.T @ H, da.sum(axis=0), a.T @ g, float(g.sum())"),
 ("        if db[b] <= rel < de[b]:", "        if True:"),
 # decode
 ("            x = scale * (K[lo:lo + n, kv] @ Q[b, h]) + g[h] * s[lo:lo + n]", "            x = scale * (K[lo:lo + n, kv] @ Q[b, h])"),
 ("            lse[b, h] = m + math.log(e.sum())", "            lse[b, h] = math.log(e.sum())"),
 ("        lo, n = int(start[b]), int(lens[b])\n        if n == 0:\n            continue\n        for h in range(Hq):\n            kv = h // group\n            x = scale * (K[lo:lo + n, kv]", "        lo, n = int(start[b]), int(lens[b]) - 1\n        if n <= 0:\n            continue\n        for h in range(Hq):\n            kv = h // group\n            x = scale * (K[lo:lo + n, kv]"),
 # more selection / compaction
 ("        keep[lo:hi] = 1\n", ""),
 ("    kept_idx = np.nonzero(keep)[0].astype(np.int64)", "    kept_idx = np.nonzero(keep)[0].astype(np.int64)[::-1]"),
 ("    hidden_k = np.asarray(hidden)[kept_idx]", "    hidden_k = np.asarray(hidden)[kept_idx - 1]"),
 # more layer
 ("    v = y[:, (Hq + Hkv) * d:].reshape(n, Hkv, d)", "    v = y[:, Hq * d:(Hq + Hkv) * d].reshape(n, Hkv, d)"),
 ("    return apply_rope(q, pos, theta), apply_rope(k, pos, theta), v", "    return apply_rope(q, np.arange(n), theta), apply_rope(k, np.arange(n), theta), v"),
 ("    o, _ = gated_attention(q, k, v, bias, gain, tau, cu_kept, rows=rows)", "    o, _ = gated_attention(q, k, v, None, None, tau, cu_kept, rows=rows)"),
 # more backward
 ("            dq[lo:hi, h] = scale * (dx @ Kh)", "            dq[lo:hi, h] = dx @ Kh"),
 ("        visible = np.arange(n)[None, :] <= np.arange(n)[:, None]\n        sb = s[lo:hi]", "        visible = np.arange(n)[None, :] < np.arange(n)[:, None] + (np.arange(n)[:, None] == 0)\n        sb = s[lo:hi]"),
 # more decode
 ("            kv = h // group\n            x = scale * (K[lo:lo + n, kv] @ Q[b, h])", "            kv = h % K.shape[1]\n            x = scale * (K[lo:lo + n, kv] @ Q[b, h])"),
 ("            o[b, h] = e @ V[lo:lo + n, kv] / e.sum()", "            o[b, h] = e @ V[lo:lo + n, kv] / n"),
 # backward, column form and dq rows
 ("            dk[n, kv] += scale * (dx @ Qi)", "            dk[n, kv] += dx @ Qi"),
 ("            dv[n, kv] += P @ dOi", "            dv[n, kv] += dx @ dOi"),
 ("            P = np.exp(x - L[h, j:hi])", "            P = np.exp(x - L[h, j])"),
 ("                ds[n] += g[h] * float(dx.sum())", "                ds[n] += float(dx.sum())"),
 ("            Qi, dOi = Q[j:hi, h], dO[j:hi, h]", "            Qi, dOi = Q[j + 1:hi, h], dO[j + 1:hi, h]"),
 ("            dq[i, h] = scale * (dx @ Kh)", "            dq[i, h] = scale * (dx @ Vh)"),
 ("            Kh, Vh = K[lo:i + 1, kv], V[lo:i + 1, kv]", "            Kh, Vh = K[lo:i, kv], V[lo:i, kv]"),
 # gate backward
 ("    return da @ W, da.T @ H, da.sum(axis=0), z.T @ g, float(g.sum())", "    return da @ (2.0 * W), da.T @ H, da.sum(axis=0), z.T @ g, float(g.sum())"),
 ("    return da @ W, da.T @ H, da.sum(axis=0), z.T @ g, float(g.sum())", "    return da @ W, da.T @ H, da.sum(axis=0), z.T @ g, float(g.sum()) + 1.0"),
 ("    a = H @ W.T\n    if b1 is not None:\n        a = a + _f64(b1)[None, :]\n    sig", "    a = H @ W.T\n    sig"),
 # sampling
 ("    return np.floor(f * (de - db)).astype(np.int64)", "    return np.rint(f * (de - db)).astype(np.int64)"),
 ("    f = float(min_frac) + (float(max_frac) - float(min_frac)) * uu", "    f = float(min_frac) + float(max_frac) * uu"),
]

def setup(M):
    os.makedirs(M + "/tests")
    for d in ("oracle", "synth"):
        shutil.copytree(R + "/" + d, M + "/" + d, ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copytree(R + "/tests/golden", M + "/tests/golden")
    for f in ("tests/conftest.py", "tests/test_oracle_pins.py", "pytest.ini"):
        shutil.copy(R + "/" + f, M + "/" + f)

def run(M):
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "tests/test_oracle_pins.py"],
                       cwd=M, capture_output=True, text=True)
    return r.returncode, r.stdout.strip().splitlines()[-1] if r.stdout.strip() else r.stderr[-300:]

def main():
    with tempfile.TemporaryDirectory() as tmp:
        M = os.path.join(tmp, "tree")
        setup(M)
        rc, tail = run(M)
        print("baseline:", rc, tail, flush=True)
        if rc != 0:
            return 2
        src = open(R + "/oracle/tokengate.py").read()
        survivors = []
        for i, (a, b) in enumerate(MUTS):
            n = src.count(a)
            if n != 1:
                print(f"[{i}] pattern found {n} times, skipped: {a[:60]!r}", flush=True)
                survivors.append(i)
                continue
            open(M + "/oracle/tokengate.py", "w").write(src.replace(a, b))
            rc, tail = run(M)
            status = "caught" if rc != 0 else "SURVIVED"
            print(f"[{i}] {status}: {a.strip()[:70]!r} -> {b.strip()[:50]!r} | {tail}", flush=True)
            if rc == 0:
                survivors.append(i)
        print("survivors:", survivors)
        return 1 if survivors else 0


if __name__ == "__main__":
    sys.exit(main())
