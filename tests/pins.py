"""Pins of the CPU oracle: checks against facts fixed outside the oracle.

Each check_* function raises AssertionError on a violation.  They are run on
the real oracle (test_oracle_pins.py) and on deliberately broken copies of
oracle.c (test_oracle_mutants.py), where at least one must fail.

Kinds of pins used (none re-runs the oracle's own formula):
  - hand-derived golden values (tests/golden/*.json);
  - closed forms (first AdamW step from zero moments, constant gradients,
    zero gradients, sums of squares of powers of two);
  - exact rational arithmetic (fractions.Fraction, Python big integers,
    CPython's correctly rounded int/int division) within IEEE error bounds;
  - library routines for special cases (torch's bfloat16 rounding and
    torch.optim.AdamW on the CPU, numpy float32 arithmetic);
  - exhaustive search (every bf16 pattern under every MXFP8 scale against a
    nearest-value search over the E4M3 table).
"""
import json
import math
import os
from fractions import Fraction as Fr

import numpy as np

import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
U24 = 2.0 ** -24
HYPERS = [  # (lr, beta1, beta2, eps, wd)
    (1e-3, 0.9, 0.999, 1e-8, 0.01),
    (0.1, 0.5, 0.75, 1e-3, 0.5),
    (3e-4, 0.95, 0.98, 1e-6, 0.1),
]


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def hx(s) -> int:
    return int(s, 16)


def f32_from_bits(b) -> np.float32:
    return np.array([b], dtype=np.uint32).view(np.float32)[0]


def rn32(fr: Fr) -> float:
    """Exact round-to-nearest-even of a rational to binary32."""
    c = np.float32(float(fr))
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        if not np.isfinite(cand):
            continue
        d = abs(Fr(float(cand)) - fr)
        key = (d, int(np.array([cand]).view(np.uint32)[0]) & 1)
        if best is None or key < best[0]:
            best = (key, float(cand))
    return best[1]


def ulp32(x) -> float:
    return float(np.spacing(np.float32(abs(x))))


# ------------------------------------------------------------------ bf16 ---

def check_bf16_golden():
    for c in golden("bf16_rne.json")["cases"]:
        x = f32_from_bits(hx(c["f32_bits"]))
        got = int(O.f32_to_bf16(np.array([x]))[0])
        assert got == hx(c["bf16"]), (c, hex(got))


def check_bf16_vs_torch():
    import torch
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2 ** 32, size=1 << 18, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    extra = np.array([0.0, -0.0, 1.0, np.inf, -np.inf, 3.3895314e38, -3.3895314e38,
                      1e-45, 1.17549435e-38], dtype=np.float32)
    x = np.concatenate([x, extra, (rng.standard_normal(1 << 16) * 0.02).astype(np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.f32_to_bf16(x)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(hex(int(x.view(np.uint32)[i])), hex(got[i]), hex(want[i])) for i in bad[:5]]


# --------------------------------------------------------------- scalars ---

def check_pow():
    for t in (1, 2, 3, 5, 8, 13, 64, 100, 1000, 4097):
        assert O.pow_u(0.5, t) == 2.0 ** -t
        assert O.pow_u(1.0, t) == 1.0
    for beta in (0.9, 0.999, 0.75, 0.95):
        for t in (1, 2, 3, 7, 10, 31, 100, 333):
            exact = Fr(beta) ** t
            got = Fr(O.pow_u(beta, t))
            assert abs(got - exact) <= exact * Fr(2 * t, 2 ** 53), (beta, t)


def check_scalars():
    for lr, b1, b2, eps, wd in HYPERS:
        for t in (1, 2, 3, 10, 100, 1000):
            s = O.make_scalars(lr, b1, b2, eps, wd, t)
            assert s.b1 == float(np.float32(b1)) and s.b2 == float(np.float32(b2))
            assert s.omb1 == rn32(1 - Fr(b1)), (b1, s.omb1)
            assert s.omb2 == rn32(1 - Fr(b2)), (b2, s.omb2)
            assert s.eps == float(np.float32(eps))
            bc1 = 1 - Fr(b1) ** t
            bc2 = 1 - Fr(b2) ** t
            ss = Fr(lr) / bc1
            assert abs(Fr(s.step_size) - ss) <= Fr(ulp32(float(ss))) * Fr(51, 100), (t, s.step_size)
            sq = math.sqrt(float(bc2))
            assert abs(s.sqrt_bc2 - sq) <= 0.51 * ulp32(sq) + 1e-15, (t, s.sqrt_bc2, sq)
            dec = 1 - Fr(lr) * Fr(wd)
            assert abs(Fr(s.decay) - dec) <= Fr(ulp32(float(dec))) * Fr(51, 100), (s.decay, dec)


# ---------------------------------------------------------------- reduce ---

def check_reduce_golden():
    for c in golden("reduce_order.json")["cases"]:
        if "replicas_f32" in c:
            reps = [np.array([v], dtype=np.float32) for v in c["replicas_f32"]]
        else:
            reps = [np.array([v], dtype=np.uint16) for v in c["replicas_bf16"]]
        g = O.reduce(reps, c["inv_scale"])
        assert float(g[0]) == c["g"], (c, float(g[0]))


def check_reduce_equal_replicas():
    rng = np.random.default_rng(2)
    # Values with at most 16 significant bits: every partial sum k*x (k <= 16)
    # is exact in binary32, so P equal replicas average back to x exactly.
    x = (rng.standard_normal(1000) * 0.01).astype(np.float32)
    x = (x.view(np.uint32) & np.uint32(0xFFFFFF00)).view(np.float32)
    xb = O.f32_to_bf16(x)
    for P in (1, 2, 4, 8, 16):
        g = O.reduce([x] * P, 1.0 / P)
        assert np.array_equal(g, x), P
        gb = O.reduce([xb] * P, 1.0 / P)
        assert np.array_equal(gb.view(np.uint32), (xb.astype(np.uint32) << 16)), P


def check_reduce_bound():
    rng = np.random.default_rng(3)
    n = 4096
    for P in (2, 3, 5, 8):
        reps = [(rng.standard_normal(n) * 0.01 * (k + 1)).astype(np.float32) for k in range(P)]
        inv = float(np.float32(1.0 / P))
        g = O.reduce(reps, inv).astype(np.float64)
        stack = np.stack([r.astype(np.float64) for r in reps])
        exact = np.array([math.fsum(col) for col in stack.T]) * inv
        sabs = np.abs(stack).sum(axis=0)
        bound = (0.5 * (P - 1) * np.spacing(sabs.astype(np.float32)).astype(np.float64) * inv
                 + 0.5 * np.spacing(np.abs(g).astype(np.float32)).astype(np.float64) + 1e-300)
        err = np.abs(g - exact)
        assert np.all(err <= bound * 1.0001), (P, float(np.max(err / bound)))


def check_reduce_brute_numpy():
    # 16-element vectors against numpy's binary32 arithmetic (IEEE round to
    # nearest even per operation), summed in rank order and then scaled.
    rng = np.random.default_rng(23)
    for P in (1, 2, 3, 5, 8):
        for bf16 in (False, True):
            x = [(rng.standard_normal(16) * np.exp2(rng.integers(-30, 30, size=16)))
                 .astype(np.float32) for _ in range(P)]
            reps = [O.f32_to_bf16(r) for r in x] if bf16 else x
            vals = [(r.astype(np.uint32) << 16).view(np.float32) if bf16 else r for r in reps]
            inv = np.float32(1.0 / P)
            want = np.empty(16, np.float32)
            for i in range(16):
                acc = vals[0][i]
                for k in range(1, P):
                    acc = np.float32(acc + vals[k][i])
                want[i] = np.float32(acc * inv)
            got = O.reduce(reps, float(inv))
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (P, bf16)


# ------------------------------------------------------------------ norm ---

def _acc_with_X(X: int, nonfinite: int = 0) -> "O.Acc":
    a = O.acc_zero()
    for k in range(O.ACC_WORDS):
        a.w[k] = (X >> (32 * k)) & 0xFFFFFFFF
    a.nonfinite = nonfinite
    return a


def _parse_int_product(text: str) -> int:
    """'25 * 2^128' -> 25 << 128 (integers and powers of two only)."""
    out = 1
    for part in text.split("*"):
        part = part.strip()
        if "^" in part:
            base, ex = part.split("^")
            out *= int(base) ** int(ex)
        else:
            out *= int(part)
    return out


def check_norm_golden():
    for c in golden("norm_fixed_point.json")["cases"]:
        g = np.array([float(v) for v in c["g"]] * c.get("repeat", 1), dtype=np.float32)
        a = O.norm_accumulate(g)
        X = _parse_int_product(c["X"])
        assert a.X == X, (c, a.X)
        assert a.nonfinite == c["nonfinite"], c
        assert O.acc_sumsq(a) == c["sumsq"], (c, O.acc_sumsq(a))


def check_norm_powers_of_two():
    # Sums of squares of +-2^k with a narrow exponent span are exact in every
    # binary64 partial sum, so X = sum 2^(2k+128) whatever the grouping.
    rng = np.random.default_rng(4)
    for n in (1, 16, 17, 31, 32, 33, 100, 257):
        k = rng.integers(-8, 15, size=n)
        sign = rng.choice([-1.0, 1.0], size=n)
        g = (sign * np.exp2(k.astype(np.float64))).astype(np.float32)
        a = O.norm_accumulate(g)
        X = sum(1 << int(2 * kk + 128) for kk in k)
        assert a.X == X and a.nonfinite == 0, n
        assert O.acc_sumsq(a) == X / 2 ** 128
    # the same over the whole binary32 range, one power of two per group (so
    # every group sum is exact): 2^-149 (smallest subnormal, floors to 0) up
    # to 2^127, whose square 2^254 is the top of the range
    k = np.array([-149, -126, -65, -64, -1, 0, 31, 32, 33, 63, 64, 100, 126, 127])
    g = np.zeros(32 * k.size, np.float32)
    g[::32] = np.exp2(k.astype(np.float64)).astype(np.float32)
    X = sum((1 << int(2 * kk + 128)) if 2 * kk + 128 >= 0 else 0 for kk in k)
    a = O.norm_accumulate(g)
    assert a.X == X and a.nonfinite == 0
    assert O.acc_sumsq(a) == X / 2 ** 128


def check_norm_brute():
    # Big-integer brute force of the stated grouping on tiny vectors.
    rng = np.random.default_rng(5)
    cases = [(n, (rng.standard_normal(n) * np.exp2(rng.integers(-30, 20, size=n)))
              .astype(np.float32)) for n in (16, 17, 31, 32, 33, 64, 100)]
    # magnitudes over the whole finite binary32 range, mixed within groups
    cases += [(n, (rng.standard_normal(n) * np.exp2(rng.integers(-150, 125, size=n)))
               .astype(np.float32)) for n in (16, 32, 96, 257)]
    cases.append((64, np.full(64, np.finfo(np.float32).max, np.float32)
                   * np.where(rng.random(64) < 0.5, -1, 1).astype(np.float32)))
    cases.append((2048, (rng.standard_normal(2048) * 1e-3).astype(np.float32)))
    for n, g in cases:
        X = 0
        for gs in range(0, n, 32):
            parts = []
            for j in range(4):
                s = 0.0
                for t in range(8):
                    i = gs + 8 * j + t
                    q = float(g[i]) * float(g[i]) if i < n else 0.0
                    s = s + q
                parts.append(s)
            S = (parts[0] + parts[1]) + (parts[2] + parts[3])
            X += math.floor(Fr(S) * 2 ** 128)
        a = O.norm_accumulate(g)
        assert a.X == X, n
    # group by group, so that rounding differences cannot cancel in the sum
    g = (rng.standard_normal(32 * 256) * 1e-3).astype(np.float32)
    for gs in range(0, g.size, 32):
        parts = []
        for j in range(4):
            s = 0.0
            for t in range(8):
                s = s + float(g[gs + 8 * j + t]) ** 2
            parts.append(s)
        S = (parts[0] + parts[1]) + (parts[2] + parts[3])
        assert O.norm_accumulate(g[gs:gs + 32]).X == math.floor(Fr(S) * 2 ** 128), gs


def check_norm_exact_bound():
    rng = np.random.default_rng(6)
    for n in (1000, 4096):
        g = (rng.standard_normal(n) * 0.01).astype(np.float32)
        exact = sum(Fr(float(x)) ** 2 for x in g)
        got = Fr(O.acc_sumsq(O.norm_accumulate(g)))
        assert abs(got - exact) <= exact * Fr(40, 2 ** 53) + Fr(n, 2 ** 128), n


def check_norm_split_invariance():
    rng = np.random.default_rng(7)
    n = 32 * 37 + 5
    g = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    g[100] = np.inf
    g[1000] = np.nan
    whole = O.norm_accumulate(g)
    padded = O.norm_accumulate(np.concatenate([g, np.zeros(27, np.float32)]))
    assert (whole.X, whole.nonfinite) == (padded.X, padded.nonfinite) == (whole.X, 2)
    for cut in (32, 64, 320, 32 * 36):
        a = O.norm_accumulate(g[:cut])
        O.acc_add(a, O.norm_accumulate(g[cut:]))
        assert (a.X, a.nonfinite) == (whole.X, whole.nonfinite), cut
    # carries across every digit: adding 1 to 2^k - 1 for k up to the top
    for k in (32, 64, 224, 256, 448, 480):
        a = _acc_with_X((1 << k) - 1)
        O.acc_add(a, _acc_with_X(1, 3))
        assert a.X == 1 << k and a.nonfinite == 3, k


def check_sumsq_rounding():
    rng = np.random.default_rng(8)
    Xs = [0, 1, 2 ** 53 - 1, 2 ** 53, 2 ** 53 + 1, 2 ** 54 + 2, 2 ** 54 + 6, 2 ** 224 - 1,
          2 ** 421 - 1, 2 ** 511 + 2 ** 459]
    for bits in range(1, 512, 3):
        Xs.append(int(rng.integers(0, 2 ** 62)) << max(0, bits - 62) | 1 << (bits - 1))
    for m in (2 ** 52 + 1, 2 ** 52 + 2, 2 ** 53 - 1):       # exact ties
        for sh in (0, 5, 100):
            Xs.append(((2 * m + 1) << sh))
            Xs.append(((2 * m + 1) << sh) + 1)
    for X in Xs:
        X &= (1 << 512) - 1
        got = O.acc_sumsq(_acc_with_X(X))
        want = Fr(X, 2 ** 128)
        # CPython's int/int division is correctly rounded where it does not
        # overflow; past binary64's range compare with exact rationals
        if X < 2 ** 1000:
            assert got == X / 2 ** 128, hex(X)
        assert abs(Fr(got) - want) <= Fr(math.ulp(got)) / 2, hex(X)


def check_clip_coef():
    assert O.clip_coef(4.0, 0.0) == 1.0 and O.clip_coef(4.0, -1.0) == 1.0
    for sumsq in (0.0, 1e-14, 0.25, 1.0, 4.0, 17.3, 1e4, 3.7e9):
        for mx in (0.5, 1.0, 2.5):
            c = O.clip_coef(sumsq, mx)
            ref = mx / (math.sqrt(sumsq) + 1e-6)
            if ref >= 1.0:
                assert c == 1.0, (sumsq, mx, c)
            else:
                assert abs(c - ref) <= 0.5 * ulp32(ref) * 1.0001, (sumsq, mx, c, ref)


# ----------------------------------------------------------------- AdamW ---

def _first_step(theta0, g, lr, b1, b2, eps, wd):
    n = len(g)
    master = np.ascontiguousarray(theta0, dtype=np.float32).copy()
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    p = np.zeros(n, np.uint16)
    O.adamw(np.asarray(g, np.float32), 1.0, O.make_scalars(lr, b1, b2, eps, wd, 1),
            master, m, v, p)
    return master, m, v, p


def check_adamw_golden():
    for c in golden("adamw_closed_form.json")["cases"]:
        master, *_ = _first_step([c["theta0"]], [c["g"]], c["lr"], c["beta1"], c["beta2"],
                                 c["eps"], c["wd"])
        want = float(c["theta1"])
        tol = 10 * U24 * (abs(c["theta0"]) + c["lr"])
        assert abs(float(master[0]) - want) <= tol, (c, float(master[0]))


def check_adamw_first_step():
    import torch
    rng = np.random.default_rng(9)
    n = 2048
    for lr, b1, b2, eps, wd in HYPERS:
        theta0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
        g = (rng.standard_normal(n) * np.exp2(rng.integers(-12, 0, size=n))).astype(np.float32)
        master, m, v, p = _first_step(theta0, g, lr, b1, b2, eps, wd)
        t0 = theta0.astype(np.float64)
        gd = g.astype(np.float64)
        upd = lr * gd / (np.abs(gd) + eps)
        want = t0 * (1 - lr * wd) - upd
        tol = 12 * U24 * (np.abs(t0) + np.abs(upd)) + 1e-30
        assert np.all(np.abs(master - want) <= tol), (lr, float(np.max(np.abs(master - want) / tol)))
        assert np.all(np.abs(m - (1 - b1) * gd) <= 3 * U24 * np.abs((1 - b1) * gd))
        assert np.all(np.abs(v - (1 - b2) * gd * gd) <= 5 * U24 * (1 - b2) * gd * gd + 1e-44)
        pb = torch.from_numpy(master).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(p, pb)


def check_adamw_constant_grad():
    rng = np.random.default_rng(10)
    n = 512
    for lr, b1, b2, eps, _ in HYPERS:
        theta0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
        g = (rng.standard_normal(n) * 1e-2).astype(np.float32)
        master, m, v = theta0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
        gd = g.astype(np.float64)
        per = lr * gd / (np.abs(gd) + eps)
        for t in range(1, 21):
            O.adamw(g, 1.0, O.make_scalars(lr, b1, b2, eps, 0.0, t), master, m, v)
            want = theta0.astype(np.float64) - t * per
            tol = t * 24 * U24 * (np.abs(theta0) + np.abs(per)) + 1e-30
            assert np.all(np.abs(master - want) <= tol), (lr, t, float(np.max(np.abs(master - want) / tol)))


def check_adamw_zero_grad():
    rng = np.random.default_rng(11)
    n = 300
    for lr, b1, b2, eps, wd in HYPERS:
        theta = (rng.standard_normal(n) * 0.02).astype(np.float32)
        master, m, v = theta.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
        g = np.zeros(n, np.float32)
        for t in range(1, 8):
            s = O.make_scalars(lr, b1, b2, eps, wd, t)
            O.adamw(g, 1.0, s, master, m, v)
            theta = (theta * np.float32(s.decay)).astype(np.float32)
            assert np.array_equal(master, theta) and not m.any() and not v.any(), t


def check_adamw_vs_torch():
    import torch
    rng = np.random.default_rng(12)
    n = 4096
    for lr, b1, b2, eps, wd in HYPERS:
        theta0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
        grads = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for _ in range(10)]
        p = torch.nn.Parameter(torch.from_numpy(theta0.copy()))
        opt = torch.optim.AdamW([p], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd,
                                foreach=False)
        master, m, v = theta0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
        for t, g in enumerate(grads, 1):
            p.grad = torch.from_numpy(g.copy())
            opt.step()
            O.adamw(g, 1.0, O.make_scalars(lr, b1, b2, eps, wd, t), master, m, v)
            ref = p.detach().numpy().astype(np.float64)
            tol = t * (24 * U24 * lr + 4 * U24 * np.abs(ref))
            err = np.abs(master - ref)
            assert np.all(err <= tol), (lr, t, float(np.max(err / tol)))
            st = opt.state[p]
            gmax = max(float(np.abs(gg).max()) for gg in grads)
            assert np.all(np.abs(m - st["exp_avg"].numpy()) <= t * 4 * U24 * gmax)
            assert np.allclose(v, st["exp_avg_sq"].numpy(), rtol=t * 16 * U24, atol=1e-45)


def _rn32_sqrt(x: float) -> float:
    """Correctly rounded binary32 square root of a non-negative binary32 x,
    by exact comparison of x with the squares of candidate midpoints."""
    X = Fr(x)
    c = np.float32(math.sqrt(x))
    cands = sorted({float(v) for v in (np.nextafter(c, np.float32(-1)), c,
                                       np.nextafter(c, np.float32(np.inf))) if v >= 0})
    best = cands[0]
    for cand in cands[1:]:
        mid = (Fr(best) + Fr(cand)) / 2
        if X > mid * mid:
            best = cand
    return best


def _adamw_exact_element(g, coef, s, theta, m, v):
    """One element of the AdamW sequence in exact rational arithmetic with one
    binary32 round-to-nearest-even after every operation (fma: one rounding of
    the exact a*b + c)."""
    F = lambda x: Fr(float(x))
    gc = rn32(F(g) * F(coef))
    mi = rn32(F(s.b1) * F(m) + F(rn32(F(s.omb1) * F(gc))))
    t2 = rn32(F(s.omb2) * F(gc))
    vi = rn32(F(s.b2) * F(v) + F(rn32(F(t2) * F(gc))))
    d = rn32(F(_rn32_sqrt(vi)) / F(s.sqrt_bc2))
    d = rn32(F(d) + F(s.eps))
    u = rn32(F(mi) / F(d))
    th = rn32(F(theta) * F(s.decay))
    th = rn32(-F(s.step_size) * F(u) + F(th))
    return th, mi, vi


def check_adamw_exact_brute_ieee_corners():
    # 16-element vectors of finite IEEE corner values -- zeros of both signs,
    # subnormal gradients and state, the edges of the normal range, large
    # values short of overflow -- with beta1 = 0, full decay (lr * wd = 1)
    # and clip coefficients down to a subnormal one: every binary32 result
    # equals the exact simulation (which rounds subnormals exactly).
    rng = np.random.default_rng(25)
    n = 16
    G = [0.0, -0.0, 1e-45, -1e-45, 1e-40, -3e-39, 1.1754942e-38, 1.17549435e-38, 1e-30,
         -1e-20, 1e-3, -0.5, 1.0, 1e15, -3e15]
    TH = [0.0, -0.0, 1e-45, -1e-40, 1.17549435e-38, 0.02, -1.5, 1e30]
    M = [0.0, -0.0, 1e-45, -1e-40, 1e-30, 1e-3, -0.2, 1e20]
    V = [0.0, 1e-45, 1e-40, 1.17549435e-38, 1e-20, 1e-6, 1.0, 1e30]
    hypers = [(1e-3, 0.9, 0.999, 1e-8, 0.01), (0.1, 0.0, 0.5, 1e-6, 0.0),
              (1.0, 0.999, 0.0, 1e-6, 1.0)]
    for lr, b1, b2, eps, wd in hypers:
        master = rng.choice(np.array(TH, np.float32), n)
        mm = rng.choice(np.array(M, np.float32), n)
        vv = rng.choice(np.array(V, np.float32), n)
        param = np.zeros(n, np.uint16)
        for t, coef in ((1, 1.0), (2, 0.37), (5, float(np.float32(1e-40))), (6, 0.0)):
            g = rng.choice(np.array(G, np.float32), n)
            s = O.make_scalars(lr, b1, b2, eps, wd, t)
            want = [_adamw_exact_element(g[i], np.float32(coef), s, master[i], mm[i], vv[i])
                    for i in range(n)]
            O.adamw(g, coef, s, master, mm, vv, param)
            assert np.isfinite(master).all() and np.isfinite(mm).all() and np.isfinite(vv).all()
            for i, (th, mi, vi) in enumerate(want):
                assert (master[i], mm[i], vv[i]) == (np.float32(th), np.float32(mi),
                                                     np.float32(vi)), (lr, t, i)


def check_adamw_exact_brute():
    # 16-element vectors over several steps with nonzero moments and a clip
    # coefficient: every binary32 result equals the exact simulation, and the
    # bf16 param is torch's rounding of the new master.
    import torch
    rng = np.random.default_rng(24)
    n = 16
    for lr, b1, b2, eps, wd in HYPERS:
        theta = (rng.standard_normal(n) * 0.02).astype(np.float32)
        m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
        v = (np.abs(rng.standard_normal(n)) * 1e-7 + 1e-12).astype(np.float32)
        master, mm, vv = theta.copy(), m.copy(), v.copy()
        param = np.zeros(n, np.uint16)
        for t, coef in ((1, 1.0), (2, 0.37), (3, 1.0), (7, 0.011)):
            g = (rng.standard_normal(n) * np.exp2(rng.integers(-20, 2, size=n))).astype(np.float32)
            g[0] = np.float32(3e-30)              # products in the subnormal range
            s = O.make_scalars(lr, b1, b2, eps, wd, t)
            want = [_adamw_exact_element(g[i], np.float32(coef), s, master[i], mm[i], vv[i])
                    for i in range(n)]
            O.adamw(g, coef, s, master, mm, vv, param)
            for i, (th, mi, vi) in enumerate(want):
                assert (master[i], mm[i], vv[i]) == (np.float32(th), np.float32(mi),
                                                     np.float32(vi)), (lr, t, i)
            pb = torch.from_numpy(master).to(torch.bfloat16).view(torch.int16).numpy()
            assert np.array_equal(param, pb.view(np.uint16))


# ------------------------------------------------------ composed step ---

def check_step_clip_closed_form():
    # P equal bf16 replicas of g = [3, 4, 0, ...] * 2^-4: averaged grad is
    # exact, ||g|| = 5/16, clip coefficient c = 0.1 / (5/16 + 1e-6).
    n = 64
    gv = np.zeros(n, np.float32)
    gv[0], gv[1] = 3 / 16, 4 / 16
    reps = [O.f32_to_bf16(gv)] * 4
    theta0 = np.full(n, 0.5, np.float32)
    lr, b1, b2, eps, wd = 0.01, 0.9, 0.999, 1e-8, 0.1
    master, m, v = theta0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    skipped, acc = O.step(reps, 0.25, 0.1, True, lr, b1, b2, eps, wd, 1, master, m, v)
    assert not skipped and acc.X == (25 << 128) // 256
    c = 0.1 / (5 / 16 + 1e-6)
    gc = gv.astype(np.float64) * c
    want = 0.5 * (1 - lr * wd) - lr * gc / (np.abs(gc) + eps)
    assert np.all(np.abs(master - want) <= 12 * U24 * (0.5 + lr)), master[:2]
    assert abs(m[0] - 0.1 * gc[0]) <= 4 * U24 * abs(0.1 * gc[0])


def check_step_skip():
    rng = np.random.default_rng(13)
    n = 96
    reps = [O.f32_to_bf16((rng.standard_normal(n) * 1e-3).astype(np.float32)) for _ in range(2)]
    reps[1][n - 1] = 0x7F80  # +inf in the last element of rank 1's replica
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32)
    p = O.f32_to_bf16(master)
    before = [a.copy() for a in (master, m, v, p)]
    skipped, acc = O.step(reps, 0.5, 1.0, True, 1e-3, 0.9, 0.999, 1e-8, 0.01, 3,
                          master, m, v, p)
    assert skipped and acc.nonfinite == 1
    for a, b in zip((master, m, v, p), before):
        assert np.array_equal(a, b)
    skipped, _ = O.step(reps, 0.5, 0.0, False, 1e-3, 0.9, 0.999, 1e-8, 0.01, 3,
                        master, m, v, p)
    assert not skipped
    assert np.isfinite(master[:-1]).all() and not np.isfinite(master[-1])


def check_gate_rules():
    # The gate as a table over (nonfinite, check, max_norm): a skip only with
    # the check on; an infinite norm (a non-finite element) clips to 0; no
    # clipping gives 1; otherwise the finite clip formula.
    X = 25 << 128                       # sum of squares 25, norm 5
    for nf in (0, 1, 7):
        for check in (False, True):
            for mx in (0.0, -1.0, 1.0, 10.0):
                skip, coef = O.gate(_acc_with_X(X, nf), mx, check)
                if check and nf:
                    assert skip, (nf, check, mx)
                    continue
                assert not skip, (nf, check, mx)
                if mx <= 0:
                    want = 1.0
                elif nf:
                    want = 0.0
                else:
                    want = min(1.0, float(np.float32(mx / (5.0 + 1e-6))))
                assert coef == want, (nf, check, mx, coef)
    # an exact zero norm with clipping on is no clip at all
    assert O.gate(_acc_with_X(0), 1.0, True) == (False, 1.0)


def check_step_huge_finite_grad_is_clipped():
    # Every finite group counts toward the norm: g = 2^32 in 64 elements has
    # sum of squares 2^70 and norm 2^35, so with max_norm 1 the clipped
    # gradient is 2^32 * f32(1 / (2^35 + 1e-6)) ~ 1/8, and the first step is
    # the closed form theta0 * (1 - lr*wd) - lr * g'/(|g'| + eps).
    n = 64
    big = [np.full(n, 2.0 ** 32, np.float32)]
    theta0 = np.full(n, 0.25, np.float32)
    lr, wd, eps = 1e-3, 0.01, 1e-8
    master, m, v = theta0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    skipped, acc = O.step(big, 1.0, 1.0, True, lr, 0.9, 0.999, eps, wd, 1, master, m, v)
    assert not skipped and acc.nonfinite == 0 and acc.X == 1 << (70 + 128)
    coef = float(np.float32(1.0 / (2.0 ** 35 + 1e-6)))
    gc = 2.0 ** 32 * coef
    want = 0.25 * (1 - lr * wd) - lr * gc / (gc + eps)
    assert np.all(np.abs(master - want) <= 12 * U24 * (0.25 + lr)), master[:2]
    assert np.all(np.abs(m - 0.1 * gc) <= 4 * U24 * 0.1 * gc)


def check_step_clip_only_nonfinite():
    # Clipping on, the check off: one infinite element makes the global norm
    # infinite and the coefficient 0, so every finite element steps with a
    # zero gradient (m = v = 0, theta = theta * decay) and the infinite one
    # turns its own state into NaN (inf * 0).
    rng = np.random.default_rng(19)
    n = 96
    reps = [O.f32_to_bf16((rng.standard_normal(n) * 1e-3).astype(np.float32)) for _ in range(2)]
    reps[0][40] = 0x7F80
    master = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
    s = O.make_scalars(1e-3, 0.9, 0.999, 1e-8, 0.01, 1)
    want = (master * np.float32(s.decay)).astype(np.float32)
    skipped, acc = O.step(reps, 0.5, 1.0, False, 1e-3, 0.9, 0.999, 1e-8, 0.01, 1, master, m, v)
    assert not skipped and acc.nonfinite == 1
    keep = np.arange(n) != 40
    assert np.array_equal(master[keep], want[keep])
    assert not m[keep].any() and not v[keep].any()
    assert np.isnan(master[40]) and np.isnan(m[40]) and np.isnan(v[40])


# ------------------------------------------------------------ invariants ---

def _synthetic_replicas(rng, P, N, sigma=1e-3, outliers=True):
    reps = []
    for _ in range(P):
        x = rng.standard_normal(N) * sigma
        if outliers:
            x = np.where(rng.random(N) < 0.01, x * 100, x)
        reps.append(O.f32_to_bf16(x.astype(np.float32)))
    return reps


def check_sharded_equals_unsharded():
    # Reduce-scatter then all-gather equals all-reduce: P ranks each stepping
    # their own shard (with the other ranks' norm accumulators added) give,
    # concatenated, bit for bit the single-rank step on the full vector with
    # the same fixed-order averaged gradient.
    rng = np.random.default_rng(15)
    for P in (1, 2, 4, 8):
        for max_norm in (0.0, 1.0, 0.05):
            _identity_case(rng, P, 32 * 8 * 16, max_norm, lambda n: _synthetic_replicas(rng, P, n))
            # N = 16: every shard is shorter than one norm group, so the
            # groups of the shards are not those of the whole vector; with
            # gradients k * 2^-10 (|k| < 128, exact in bf16) every binary64
            # partial sum of squares is exact, so the norm is grouping-free
            # and the identity holds with clipping too
            _identity_case(rng, P, 16, max_norm, lambda n: [
                O.f32_to_bf16((rng.integers(-127, 128, size=n) * 2.0 ** -10)
                              .astype(np.float32)) for _ in range(P)])


def _identity_case(rng, P, N, max_norm, make_reps, steps=(1, 2, 3)):
    hp = (1e-3, 0.9, 0.999, 1e-8, 0.01)
    S = N // P
    master0 = (rng.standard_normal(N) * 0.02).astype(np.float32)
    full = [master0.copy(), np.zeros(N, np.float32), np.zeros(N, np.float32),
            O.f32_to_bf16(master0)]
    shard = [a.copy() for a in full]
    for t in steps:
        reps = make_reps(N)
        inv = O.inv_scale(P, 1.0)
        g = O.reduce(reps, inv)
        O.step([g], 1.0, max_norm, True, *hp, t, *full)
        accs = [O.norm_accumulate(O.reduce([r[i * S:(i + 1) * S] for r in reps], inv))
                for i in range(P)]
        for i in range(P):
            sl = slice(i * S, (i + 1) * S)
            views = [a[sl] for a in shard]
            others = [accs[j] for j in range(P) if j != i]
            O.step([r[sl] for r in reps], inv, max_norm, True, *hp, t, *views,
                   extra_accs=others)
        for a, b in zip(full, shard):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (P, N, max_norm, t)


def check_sharded_equals_unsharded_gpt2_size():
    # The identity at the GPT-2-small-sized vector (N = 124,439,808, P = 8,
    # shards of 15,554,976), clip 1.0, two steps, on the workload's own
    # synthetic gradients (1 % outliers x 100): the unsharded step spread
    # over threads against the 8 shard steps with the other ranks' norm
    # states added.
    from concurrent.futures import ThreadPoolExecutor
    import synth
    from synth import configs
    w = configs.GPT2_SMALL
    N, P, S = w.N, w.P, w.S
    threads = min(8, os.cpu_count() or 1)
    hp = (w.lr, w.beta1, w.beta2, w.eps, w.wd)
    master0 = synth.fill(w.master_spec(), 0, N, False, threads=threads)
    full = [master0, np.zeros(N, np.float32), np.zeros(N, np.float32), O.f32_to_bf16(master0)]
    shard = [a.copy() for a in full]
    inv = O.inv_scale(P, 1.0)
    g_tmp = np.empty(N, np.float32)
    with ThreadPoolExecutor(threads) as ex:
        for t in (1, 2):
            reps = [synth.fill(w.grad_spec(t, k), 0, N, True, threads=threads) for k in range(P)]
            skipped, _ = O.step_parallel(reps, inv, w.max_norm, True, *hp, t, *full,
                                         g_tmp=g_tmp, threads=threads)
            assert not skipped
            sl = [slice(i * S, (i + 1) * S) for i in range(P)]
            accs = list(ex.map(lambda i: O.norm_accumulate(O.reduce([r[sl[i]] for r in reps],
                                                                    inv)), range(P)))

            def rank(i):
                others = [accs[j] for j in range(P) if j != i]
                return O.step([r[sl[i]] for r in reps], inv, w.max_norm, True, *hp, t,
                              *[a[sl[i]] for a in shard], extra_accs=others,
                              g_tmp=g_tmp[sl[i]])[0]
            assert not any(ex.map(rank, range(P)))
            del reps
            for a, b in zip(full, shard):
                assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), t


def check_loss_scale_invariance():
    # Gradients scaled by 2^16 (exact in bf16) and unscaled by inv_scale give
    # the same step bit for bit.
    rng = np.random.default_rng(16)
    N, P = 1024, 4
    reps = _synthetic_replicas(rng, P, N, outliers=False)
    scaled = [(r.astype(np.uint32) + (16 << 7)).astype(np.uint16) for r in reps]
    for r, s in zip(reps, scaled):
        assert np.array_equal(O.bf16_to_f32(s), O.bf16_to_f32(r) * np.float32(65536))
    states = []
    for rr, ls in ((reps, 1.0), (scaled, 65536.0)):
        master = (np.random.default_rng(17).standard_normal(N) * 0.02).astype(np.float32)
        st = [master, np.zeros(N, np.float32), np.zeros(N, np.float32), O.f32_to_bf16(master)]
        O.step(rr, O.inv_scale(P, ls), 1.0, True, 1e-3, 0.9, 0.999, 1e-8, 0.01, 1, *st)
        states.append(st)
    for a, b in zip(*states):
        assert np.array_equal(a, b)


def check_skip_then_continue():
    # A skipped call leaves no trace: the run G1, G_inf (skipped), G2 equals
    # the run G1, G2, with the step counter not advanced by the skip.
    rng = np.random.default_rng(18)
    N, P = 512, 2
    G1, G2 = _synthetic_replicas(rng, P, N), _synthetic_replicas(rng, P, N)
    Ginf = _synthetic_replicas(rng, P, N)
    Ginf[0][N // 3] = 0x7F80
    master = (rng.standard_normal(N) * 0.02).astype(np.float32)
    hp = (1e-3, 0.9, 0.999, 1e-8, 0.01)
    runs = []
    for seq in ((G1, G2), (G1, Ginf, G2)):
        st = [master.copy(), np.zeros(N, np.float32), np.zeros(N, np.float32),
              O.f32_to_bf16(master)]
        t = 1
        for G in seq:
            skipped, _ = O.step(G, 0.5, 1.0, True, *hp, t, *st)
            t += 0 if skipped else 1
        runs.append((st, t))
    assert runs[0][1] == runs[1][1] == 3
    for a, b in zip(runs[0][0], runs[1][0]):
        assert np.array_equal(a, b)


# ----------------------------------------------------------------- MXFP8 ---

def _e4m3_table():
    vals = []
    for code in range(0x7F):
        e, mt = code >> 3, code & 7
        vals.append(mt * 2.0 ** -9 if e == 0 else (8 + mt) * 2.0 ** (e - 10))
    return np.array(vals)


def _nearest_e4m3(q: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code by search; ties to the even code; saturating."""
    tab = _e4m3_table()
    a = np.abs(q)
    hi = np.clip(np.searchsorted(tab, a, side="left"), 0, len(tab) - 1)
    lo = np.clip(hi - 1, 0, None)
    dl = np.abs(a - tab[lo])
    dh = np.abs(tab[hi] - a)
    pick = np.where(dl < dh, lo, np.where(dh < dl, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(a >= tab[-1], len(tab) - 1, pick)
    return (pick | np.where(np.signbit(q), 0x80, 0)).astype(np.uint8)


def check_e4m3_table():
    for code in range(256):
        val = O.e4m3_value(code)
        if code & 0x7F == 0x7F:
            assert math.isnan(val)
            continue
        assert O.e4m3_encode(val) == code or (val == 0 and code in (0, 0x80))


def check_mx_exhaustive():
    x = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = (x & 0x7F80) != 0x7F80
    x = x[finite]
    xv = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for e_s in range(-127, 128):
        got = O.mx_encode_array(x, e_s)
        want = _nearest_e4m3(np.ldexp(xv, -e_s))
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (e_s, [(hex(int(x[i])), hex(got[i]), hex(want[i])) for i in bad[:4]])


def check_mx_golden():
    for b in golden("mxfp8_blocks.json")["blocks"]:
        fill = hx(b.get("fill", "0x0000"))
        blk = np.full(32, fill, np.uint16)
        blk[:len(b["bf16"])] = [hx(v) for v in b["bf16"]]
        elem, scale = O.mxfp8_pack(blk)
        assert int(scale[0]) == hx(b["scale"]), (b, int(scale[0]))
        want = np.full(32, hx(b.get("codes_fill", "0x00")), np.uint8)
        want[:len(b["codes"])] = [hx(v) for v in b["codes"]]
        assert np.array_equal(elem, want), (b, [hex(v) for v in elem[:8]])


def check_mx_block_properties():
    rng = np.random.default_rng(14)
    x = O.f32_to_bf16((rng.standard_normal(32 * 512) * np.repeat(
        np.exp2(rng.integers(-40, 40, size=512)), 32)).astype(np.float32))
    elem, scale = O.mxfp8_pack(x)
    xv = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64).reshape(-1, 32)
    for b in range(512):
        amax = np.max(np.abs(xv[b]))
        e_s = int(scale[b]) - 127
        assert 2.0 ** (e_s + 8) <= amax < 2.0 ** (e_s + 9), b
        dec = np.array([O.e4m3_value(int(c)) for c in elem[32 * b:32 * b + 32]]) * 2.0 ** e_s
        # every element within half a quantum of its E4M3 binade, or saturated
        assert np.all(np.abs(dec - xv[b]) <= np.maximum(np.abs(xv[b]) * 2.0 ** -4,
                                                       2.0 ** (e_s - 10)) + 64 * 2.0 ** e_s)


def check_mx_decode_vs_torch_fp8():
    # Element values from torch's float8_e4m3fn (a library routine), scaled
    # by 2^(scale-127) exactly in binary64 and rounded once to binary32.
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().double().numpy()
    for sb in list(range(0, 256, 7)) + [1, 126, 127, 128, 254, 255]:
        elem = np.tile(codes, 1)
        scale = np.full(256 // 32, sb, np.uint8)
        got = O.mxfp8_decode(elem, scale)
        if sb == 0xFF:
            assert np.isnan(got).all()
            continue
        want = np.ldexp(ref, sb - 127).astype(np.float32)
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(got), nan), sb
        assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32)), sb
        assert np.array_equal(np.signbit(got[nan]), codes[nan] >= 0x80)


def check_mx_decode_golden_and_roundtrip():
    for b in golden("mxfp8_blocks.json")["blocks"]:
        if b["scale"] in ("0xFF",):
            continue
        fill = hx(b.get("fill", "0x0000"))
        blk = np.full(32, fill, np.uint16)
        blk[:len(b["bf16"])] = [hx(v) for v in b["bf16"]]
        elem, scale = O.mxfp8_pack(blk)
        dec = O.mxfp8_decode(elem, scale).astype(np.float64)
        x = (blk.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        e_s = int(scale[0]) - 127
        # each element decodes to within half an E4M3 step of its input, or to
        # +-448 * 2^e_s when it saturated
        step = np.where(np.abs(x) < 2.0 ** (e_s - 6), 2.0 ** (e_s - 9),
                        2.0 ** (np.floor(np.log2(np.maximum(np.abs(x), 1e-300))) - 3))
        sat = np.abs(x) >= 448 * 2.0 ** e_s
        ok = np.where(sat, np.abs(dec) == 448 * 2.0 ** e_s, np.abs(dec - x) <= step / 2)
        assert ok.all(), (b, dec[:4], x[:4])
    # hand values: 1.0, 0.94140625, 0.96875, 0.90625 under scale byte 119
    elem = np.zeros(32, np.uint8)
    elem[:4] = [0x78, 0x77, 0x78, 0x76]
    dec = O.mxfp8_decode(elem, np.array([0x77], np.uint8))
    assert list(dec[:4]) == [1.0, 0.9375, 1.0, 0.875]
    # subnormal codes at the smallest scale: 3 * 2^-9 * 2^-127 = 3 * 2^-136
    dec = O.mxfp8_decode(np.full(32, 0x83, np.uint8), np.array([0], np.uint8))
    assert dec[0] == -3 * 2.0 ** -136


def check_mx_sizes():
    # Bytes per weight: bf16 2, MXFP8 1 + 1/32.  Stored state of 16 B per
    # weight with param and grad in MXFP8 shrinks by 12.1 %, and an
    # all-gathered bf16 payload by 48.4 % ("half").
    n = 32 * 1000
    elem, scale = O.mxfp8_pack(np.zeros(n, np.uint16))
    per = (elem.nbytes + scale.nbytes) / n
    assert per == 1.03125
    stored = (2 * (2 - per)) / 16
    wire = 1 - per / 2
    assert round(100 * stored) == 12 and abs(wire - 0.5) < 0.02
    assert 2 + 2 + 4 + 4 + 4 == 16            # bf16 p, bf16 g, fp32 master, m, v
    assert round(30e9 * 16 / 2 ** 30) == 447   # the 30B example's state per copy


ALL = [v for k, v in sorted(globals().items()) if k.startswith("check_")]
_SLOW = ("check_mx_exhaustive", "check_adamw_vs_torch", "check_bf16_vs_torch",
         "check_sharded_equals_unsharded", "check_sharded_equals_unsharded_gpt2_size")
ALL_CHEAP_FIRST = ([c for c in ALL if c.__name__ not in _SLOW]
                   + [c for c in ALL if c.__name__ in _SLOW])
