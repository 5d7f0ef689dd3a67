"""Pins for the CPU oracle: each check compares the oracle with something that
is not the oracle -- hand-derived fixtures (tests/golden), exact rational
brute force, closed forms, invariants, and library routines (torch's bf16
conversions, numpy's float64/int64 matmul, Python's sorted()).

Every check takes an ``oracle.Oracle`` and raises AssertionError on a
mismatch.  The same checks run against deliberately broken copies of the
oracle source (tests/test_oracle_mutations.py), which shows that a plausible
slip in the oracle -- a transposed operand, a dropped term, a wrong rounding
tie, an unstable ordering -- fails at least one of them.
"""
from __future__ import annotations

import ast
import bisect
import math
import operator
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# ---------------------------------------------------------------- helpers


def exact(expr: str) -> Fraction:
    """Parse an exact arithmetic expression ('1+3*2^-8', '201/64') into a Fraction."""
    ops = {ast.Add: operator.add, ast.Sub: operator.sub, ast.Mult: operator.mul,
           ast.Div: operator.truediv, ast.Pow: operator.pow}

    def ev(node):
        if isinstance(node, ast.Expression):
            return ev(node.body)
        if isinstance(node, ast.Constant) and isinstance(node.value, int):
            return Fraction(node.value)
        if isinstance(node, ast.UnaryOp) and isinstance(node.op, ast.USub):
            return -ev(node.operand)
        if isinstance(node, ast.BinOp) and type(node.op) in ops:
            left, right = ev(node.left), ev(node.right)
            if isinstance(node.op, ast.Pow):
                assert right.denominator == 1
                return left ** int(right)
            return ops[type(node.op)](left, right)
        raise ValueError(f"unsupported expression {expr!r}")

    return ev(ast.parse(expr.replace("^", "**"), mode="eval"))


def read_table(name: str):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def torch_bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Library decode: torch's bfloat16 -> float64 conversion."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def torch_f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Library rounding: torch's float32 -> bfloat16 conversion (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bits_of(values, dtype=torch.float32) -> np.ndarray:
    """bf16 bit patterns of exactly representable values (library conversion)."""
    t = torch.tensor(values, dtype=dtype).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def random_bf16(shape, seed: int, sigma: float = 1.0) -> np.ndarray:
    g = torch.Generator().manual_seed(seed)
    v = torch.randn(tuple(shape), generator=g) * sigma
    return v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def random_int_bf16(shape, seed: int, lo: int = -4, hi: int = 4) -> np.ndarray:
    g = torch.Generator().manual_seed(seed)
    v = torch.randint(lo, hi + 1, tuple(shape), generator=g).to(torch.float32)
    return v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def values(bits: np.ndarray) -> np.ndarray:
    return torch_bf16_to_f64(bits)


_FINITE_POS = None


def finite_positive_bf16():
    """(exact Fraction values, bit patterns) of all finite bf16 >= 0, ascending."""
    global _FINITE_POS
    if _FINITE_POS is None:
        bits = np.arange(0, 0x7F80, dtype=np.uint16)  # 0 .. largest finite
        vals = torch_bf16_to_f64(bits)
        _FINITE_POS = ([Fraction(float(v)) for v in vals], [int(b) for b in bits])
    return _FINITE_POS


def brute_round_bf16(v: Fraction) -> int:
    """Nearest bf16 to an exact value, ties to the even pattern, by search over all values."""
    if v < 0:
        return 0x8000 | brute_round_bf16(-v)
    vals, bits = finite_positive_bf16()
    top = vals[-1]
    # beyond the midpoint of the largest finite value and 2^128: infinity (the even neighbour)
    if v >= (top + Fraction(2) ** 128) / 2:
        return 0x7F80
    i = bisect.bisect_left(vals, v)
    if i < len(vals) and vals[i] == v:
        return bits[i]
    lo, hi = i - 1, i
    if hi >= len(vals):
        return bits[lo]
    d_lo, d_hi = v - vals[lo], vals[hi] - v
    if d_lo < d_hi:
        return bits[lo]
    if d_hi < d_lo:
        return bits[hi]
    return bits[lo] if bits[lo] % 2 == 0 else bits[hi]


def exact_projection(x_bits, W_bits):
    """Exact rational y and A by brute force over Fractions."""
    xv = [[Fraction(float(v)) for v in row] for row in values(x_bits)]
    wv = [[Fraction(float(v)) for v in row] for row in values(W_bits)]
    M, N = len(xv), len(wv)
    y = [[sum((a * b for a, b in zip(xv[m], wv[n])), Fraction(0)) for n in range(N)] for m in range(M)]
    A = [[sum((abs(a * b) for a, b in zip(xv[m], wv[n])), Fraction(0)) for n in range(N)]
         for m in range(M)]
    return y, A


def close(a, b, scale, rel, what):
    a, b, scale = np.asarray(a), np.asarray(b), np.asarray(scale)
    err = np.abs(a - b)
    bound = rel * scale
    bad = err > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} mismatches, worst err {err.max():.3e}"


# ---------------------------------------------------------------- bf16


def check_bf16_decode_golden(o):
    for row in read_table("bf16_decode.txt"):
        bits, expect = int(row[0], 16), row[1]
        got = o.c.oracle_bf16_to_f64(bits)
        if expect == "nan":
            assert math.isnan(got), (hex(bits), got)
        elif expect in ("inf", "-inf"):
            assert got == float(expect), (hex(bits), got)
        elif expect == "-0":
            assert got == 0.0 and math.copysign(1.0, got) < 0, (hex(bits), got)
        else:
            assert Fraction(got) == exact(expect), (hex(bits), got, expect)


def check_bf16_decode_all_patterns(o):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = o.bf16_to_f64(bits)
    ref = torch_bf16_to_f64(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "NaN patterns differ"
    assert np.array_equal(got[~nan], ref[~nan]), "decoded values differ from torch"
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan])), "signs differ"


def check_bf16_round_golden(o):
    for row in read_table("bf16_round.txt"):
        expr, expect = row[0], int(row[1], 16)
        if expr == "-0":
            v = -0.0
        else:
            q = exact(expr)
            v = float(q)
            if Fraction(v) != q:  # not a double: only used far from a tie
                assert expr == "314159/100000" or expr == "1/10", expr
        got = o.c.oracle_f64_to_bf16(v)
        assert got == expect, (expr, hex(got), hex(expect))


def check_bf16_round_vs_torch(o):
    rng = np.random.default_rng(11)
    # random binary32 patterns over the whole range, plus exact ties (low half 0x8000)
    words = rng.integers(0, 2 ** 32, size=20000, dtype=np.uint64).astype(np.uint32)
    ties = (words & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    near = (words & np.uint32(0xFFFF0000)) | rng.integers(0x7FF0, 0x8010, size=words.size).astype(np.uint32)
    allw = np.concatenate([words, ties, near])
    f = allw.view(np.float32)
    f = f[np.isfinite(f)]
    ref = torch_f32_to_bf16_bits(f)
    got = o.encode_bf16(f.astype(np.float64))
    bad = got != ref
    assert not bad.any(), f"{int(bad.sum())} float32 roundings differ from torch, e.g. {f[bad][:3]}"


def check_bf16_round_bruteforce(o):
    rng = np.random.default_rng(12)
    cases = []
    # doubles between bf16 neighbours (not float32 values), across normal and subnormal ranges
    for e in list(range(-140, -120)) + list(range(-20, 20)) + list(range(120, 128)):
        for _ in range(12):
            cases.append(float(np.ldexp(rng.uniform(1.0, 2.0), e)) * (1 if rng.random() < 0.5 else -1))
    # exact midpoints and midpoints +- one double ulp
    vals, _ = finite_positive_bf16()
    idx = rng.integers(1, len(vals) - 1, size=300)
    for i in idx:
        mid = (vals[i] + vals[i + 1]) / 2
        m = float(mid)
        cases += [m, math.nextafter(m, math.inf), math.nextafter(m, -math.inf)]
    for v in cases:
        got = o.c.oracle_f64_to_bf16(v)
        want = brute_round_bf16(Fraction(v))
        assert got == want, (v, hex(got), hex(want))


# ---------------------------------------------------------------- projection


def _golden_projection():
    rows = {}
    for row in read_table("projection_worked.txt"):
        rows.setdefault(row[0].rstrip(":"), []).append([exact(t) for t in row[1:]])
    return rows


def check_projection_golden(o):
    g = _golden_projection()
    x = bits_of([[float(v) for v in r] for r in g["x"]])
    W = bits_of([[float(v) for v in r] for r in g["W"]])
    y, A = o.projection(x, W)
    assert np.array_equal(y, np.array([[float(v) for v in r] for r in g["y"]])), y
    assert np.array_equal(A, np.array([[float(v) for v in r] for r in g["A"]])), A
    r = bits_of([[float(v) for v in row] for row in g["r"]])
    out = o.residual(r, y)
    assert np.array_equal(out, np.array([[float(v) for v in row] for row in g["out"]])), out


def check_projection_exact_small(o):
    for seed, (M, N, K) in enumerate([(1, 1, 1), (1, 3, 8), (2, 5, 16), (3, 4, 13), (2, 2, 7)]):
        x = random_bf16((M, K), 100 + seed)
        W = random_bf16((N, K), 200 + seed, sigma=0.02)
        y, A = o.projection(x, W)
        ye, Ae = exact_projection(x, W)
        for m in range(M):
            for n in range(N):
                # k-ascending double accumulation: error at most K * 2^-53 * A
                bound = Fraction(K) * Fraction(2) ** -52 * Ae[m][n]
                assert abs(Fraction(y[m, n]) - ye[m][n]) <= bound, (M, N, K, m, n)
                assert abs(Fraction(A[m, n]) - Ae[m][n]) <= bound, (M, N, K, m, n)


def check_projection_integer(o):
    for seed, (M, N, K) in enumerate([(1, 7, 64), (2, 9, 300), (5, 3, 1000)]):
        x = random_int_bf16((M, K), 300 + seed)
        W = random_int_bf16((N, K), 400 + seed)
        y, A = o.projection(x, W)
        xi = values(x).astype(np.int64)
        wi = values(W).astype(np.int64)
        assert np.array_equal(y, (xi @ wi.T).astype(np.float64)), (M, N, K)
        assert np.array_equal(A, (np.abs(xi) @ np.abs(wi).T).astype(np.float64)), (M, N, K)


def check_projection_vs_numpy(o):
    x = random_bf16((3, 520), 501)
    W = random_bf16((37, 520), 502, sigma=0.02)
    y, A = o.projection(x, W)
    xv, wv = values(x), values(W)
    close(y, xv @ wv.T, A, 1e-12, "y vs numpy")
    close(A, np.abs(xv) @ np.abs(wv).T, A, 1e-12, "A vs numpy")


def check_projection_layout(o):
    M, N, K = 2, 5, 9
    W = random_bf16((N, K), 601)
    for k in (0, 4, K - 1):
        x = np.zeros((M, K), dtype=np.uint16)
        x[:, k] = 0x3F80  # 1.0
        y = o.projection(x, W, with_scale=False)
        for m in range(M):
            assert np.array_equal(y[m], values(W)[:, k]), f"one-hot x picks column {k} of W"
    x = random_bf16((M, K), 602)
    picks = [3, 0, 8, 8, 5]
    Wsel = np.zeros((N, K), dtype=np.uint16)
    for n, k in enumerate(picks):
        Wsel[n, k] = 0x3F80
    y = o.projection(x, Wsel, with_scale=False)
    for n, k in enumerate(picks):
        assert np.array_equal(y[:, n], values(x)[:, k]), f"one-hot row {n} of W picks column {k} of x"


def check_projection_identity_zero(o):
    K = 11
    x = random_bf16((3, K), 701)
    eye = np.zeros((K, K), dtype=np.uint16)
    np.fill_diagonal(eye, 0x3F80)
    y = o.projection(x, eye, with_scale=False)
    assert np.array_equal(y, values(x)), "W = I gives y = x"
    zeros = np.zeros((4, K), dtype=np.uint16)
    assert not o.projection(x, zeros, with_scale=False).any(), "W = 0 gives 0"
    assert not o.projection(np.zeros((2, K), dtype=np.uint16), random_bf16((4, K), 702),
                            with_scale=False).any(), "x = 0 gives 0"


def check_projection_linearity(o):
    M, N, K = 2, 6, 64
    x = random_bf16((M, K), 801)
    W = random_bf16((N, K), 802, sigma=0.02)
    y, A = o.projection(x, W)
    for a in (-3, 5):
        xs = bits_of((values(x) * 2.0 ** a).astype(np.float32))  # exact power-of-two scaling
        ys = o.projection(xs, W, with_scale=False)
        assert np.array_equal(ys, y * 2.0 ** a), f"y(2^{a} x) = 2^{a} y(x)"
    mask = (np.arange(K) % 3 == 0)
    x1 = np.where(mask, x, 0).astype(np.uint16)
    x2 = np.where(mask, 0, x).astype(np.uint16)
    y1 = o.projection(x1, W, with_scale=False)
    y2 = o.projection(x2, W, with_scale=False)
    close(y1 + y2, y, A, 1e-13, "additivity over disjoint supports")


def check_projection_rows(o):
    M, N, K = 8, 5, 40
    x = random_bf16((M, K), 901)
    W = random_bf16((N, K), 902, sigma=0.02)
    y = o.projection(x, W, with_scale=False)
    perm = np.array([3, 7, 0, 1, 6, 2, 5, 4])
    yp = o.projection(x[perm], W, with_scale=False)
    assert np.array_equal(yp, y[perm]), "permuting x rows permutes y rows"
    y4 = o.projection(x[:4], W, with_scale=False)
    assert np.array_equal(y4, y[:4]), "a prefix of x gives the prefix of y"
    Wp = np.array([4, 2, 0, 1, 3])
    yw = o.projection(x, W[Wp], with_scale=False)
    assert np.array_equal(yw, y[:, Wp]), "permuting W rows permutes y columns"


# ---------------------------------------------------------------- split-K


def check_splitk(o):
    for (M, N, K) in [(3, 5, 40), (1, 4, 7168), (2, 3, 9), (2, 3, 2056)]:
        x = random_bf16((M, K), 1001 + K)
        W = random_bf16((N, K), 1002 + K, sigma=0.02)
        y, A = o.projection(x, W)
        xv, wv = values(x), values(W)
        for S in (1, 2, 3, 4, 7, 8, 16, 64):
            P = o.splitk_partials(x, W, S)
            assert P.shape == (S, M, N)
            close(o.splitk_sum(P), y, A, 1e-12, f"sum of partials = y (K={K}, S={S})")
            c = 64 * -(-K // (64 * S))  # ceil(K/S) rounded up to a multiple of 64
            for s in range(S):
                lo, hi = s * c, min(K, (s + 1) * c)
                if lo >= hi:
                    assert not P[s].any(), f"empty chunk {s} is 0"
                    continue
                ref = xv[:, lo:hi] @ wv[:, lo:hi].T
                scale = np.abs(xv[:, lo:hi]) @ np.abs(wv[:, lo:hi]).T
                close(P[s], ref, scale, 1e-12, f"chunk {s} of {S} covers [{lo},{hi})")


def check_splitk_sum_order(o):
    # 2^53 + 1 rounds back to 2^53 (tie to even), so s-ascending gives 0; any other order gives 1.
    P = np.array([[[2.0 ** 53]], [[1.0]], [[-(2.0 ** 53)]]])
    y = o.splitk_sum(P)
    assert y[0, 0] == 0.0, f"partials must be added in ascending s, got {y[0, 0]}"


# ---------------------------------------------------------------- residual


def check_residual(o):
    M, N, K = 3, 17, 33
    x = random_bf16((M, K), 1101)
    r = random_bf16((M, N), 1102)
    zeros = np.zeros((N, K), dtype=np.uint16)
    y = o.projection(x, zeros, with_scale=False)
    out = o.residual(r, y)
    assert np.array_equal(out, values(r)), "W = 0: residual passes r through"
    assert np.array_equal(o.encode_bf16(out), r), "W = 0: bf16 output equals r bit for bit"
    xi, wi, ri = random_int_bf16((M, K), 1103), random_int_bf16((N, K), 1104), random_int_bf16((M, N), 1105)
    y = o.projection(xi, wi, with_scale=False)
    ref = values(ri).astype(np.int64) + values(xi).astype(np.int64) @ values(wi).astype(np.int64).T
    assert np.array_equal(o.residual(ri, y), ref.astype(np.float64)), "integer residual is exact"


# ---------------------------------------------------------------- MoE table and grouped


def _golden_moe():
    cases, cur = [], None
    for row in read_table("moe_table_worked.txt"):
        if row[0] == "case":
            cur = {kv.split("=")[0]: int(kv.split("=")[1]) for kv in row[1:]}
            cases.append(cur)
        else:
            cur[row[0].rstrip(":")] = [int(v) for v in row[1:]]
    return cases


def brute_moe_table(ids: np.ndarray, E: int):
    flat = [int(v) for v in ids.ravel()]
    valid = [(e, p) for p, e in enumerate(flat) if 0 <= e < E]
    order = sorted(valid)  # by expert, then by pair index
    counts = [sum(1 for e, _ in valid if e == q) for q in range(E)]
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    pairs = [p for _, p in order] + [-1] * (len(flat) - len(order))
    return counts, offsets, pairs, len(flat) - len(valid)


def check_moe_golden(o):
    for case in _golden_moe():
        ids = np.array(case["ids"], dtype=np.int32).reshape(case["T"], case["topk"])
        counts, offsets, pairs, invalid = o.moe_table(ids, case["E"])
        assert list(counts) == case["counts"], (counts, case)
        assert list(offsets) == case["offsets"], (offsets, case)
        assert list(pairs) == case["sorted_pairs"], (pairs, case)
        assert invalid == case["invalid"][0], (invalid, case)


def check_moe_bruteforce(o):
    rng = np.random.default_rng(13)
    for T, topk, E in [(1, 8, 384), (16, 8, 384), (64, 8, 384), (5, 3, 4), (7, 2, 1)]:
        ids = np.stack([rng.permutation(E)[:topk] if topk <= E else rng.integers(0, E, topk)
                        for _ in range(T)]).astype(np.int32)
        # duplicates within a token, and ids outside [0, E)
        if T > 2:
            ids[1, :] = ids[1, 0]
            ids[2, 0] = -1
            ids[2, -1] = E
        counts, offsets, pairs, invalid = o.moe_table(ids, E)
        bc, bo, bp, bi = brute_moe_table(ids, E)
        assert list(counts) == bc and list(offsets) == bo, (T, topk, E)
        assert list(pairs) == bp and invalid == bi, (T, topk, E)
        # invariants
        assert counts.sum() == T * topk - invalid
        assert np.all(np.diff(offsets) >= 0)
        flat = ids.ravel()
        for e in range(E):
            seg = pairs[offsets[e]:offsets[e + 1]]
            assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)


def check_grouped(o):
    # exact rational brute force on a tiny routed problem, with an invalid id
    T, topk, E, N, K = 2, 3, 4, 3, 8
    x = random_bf16((T, K), 1201)
    W = random_bf16((E, N, K), 1202, sigma=0.02)
    ids = np.array([[2, 4, 3], [1, 2, -1]], dtype=np.int32)  # 4 == E and -1 are out of range
    out, A = o.grouped(x, W, ids)
    for t in range(T):
        for j in range(topk):
            e = ids[t, j]
            if not 0 <= e < E:
                assert not out[t, j].any() and not A[t, j].any(), "invalid id gives zeros"
                continue
            ye, Ae = exact_projection(x[t:t + 1], W[e])
            for n in range(N):
                bound = Fraction(K) * Fraction(2) ** -52 * Ae[0][n]
                assert abs(Fraction(out[t, j, n]) - ye[0][n]) <= bound, (t, j, n)
                assert abs(Fraction(A[t, j, n]) - Ae[0][n]) <= bound, (t, j, n)
    # integer inputs: exact against numpy int64
    T, topk, E, N, K = 5, 4, 9, 6, 96
    x = random_int_bf16((T, K), 1203)
    W = random_int_bf16((E, N, K), 1204)
    rng = np.random.default_rng(14)
    ids = np.stack([rng.permutation(E)[:topk] for _ in range(T)]).astype(np.int32)
    out = o.grouped(x, W, ids, with_scale=False)
    xi, wi = values(x).astype(np.int64), values(W).astype(np.int64)
    for t in range(T):
        for j in range(topk):
            assert np.array_equal(out[t, j], (wi[ids[t, j]] @ xi[t]).astype(np.float64)), (t, j)


def _golden_topk():
    cases, cur = [], None
    for row in read_table("router_topk_worked.txt"):
        if row[0] == "case":
            cur = {kv.split("=")[0]: int(kv.split("=")[1]) for kv in row[1:]}
            cases.append(cur)
        else:
            toks = " ".join(row[1:]).split("|")
            cur[row[0].rstrip(":")] = [t.split() for t in toks]
    return cases


def check_router_topk_golden(o):
    for c in _golden_topk():
        scores = np.array([[float(v) for v in r] for r in c["scores"]], dtype=np.float32)
        want = np.array([[int(v) for v in r] for r in c["ids"]], dtype=np.int32)
        assert scores.shape == (c["T"], c["E"]) and want.shape == (c["T"], c["k"])
        ids, top = o.router_topk(scores, c["k"])
        assert np.array_equal(ids, want), (c, ids)
        assert np.array_equal(top.view(np.uint32),
                              np.take_along_axis(scores, want, 1).view(np.uint32))


def check_router_topk_vs_sort(o):
    # numpy's stable lexicographic sort on (expert id, -score) keys, NaN as -inf
    rng = np.random.default_rng(21)
    for T, E, k in [(4, 384, 8), (3, 17, 17), (5, 64, 1), (2, 1000, 32)]:
        for kind in ("normal", "ties", "special"):
            if kind == "normal":
                s = rng.standard_normal((T, E)).astype(np.float32)
            elif kind == "ties":
                s = rng.integers(-3, 4, (T, E)).astype(np.float32)
            else:
                s = rng.integers(-2, 3, (T, E)).astype(np.float32)
                s[rng.random((T, E)) < 0.2] = np.nan
                s[rng.random((T, E)) < 0.1] = -np.inf
                s[rng.random((T, E)) < 0.05] = np.inf
            ids, top = o.router_topk(s, k)
            key = np.where(np.isnan(s), -np.inf, s).astype(np.float64)
            for t in range(T):
                order = np.lexsort((np.arange(E), -key[t]))[:k]
                assert np.array_equal(ids[t], order), (T, E, k, kind, t)
                assert len(set(ids[t].tolist())) == k


# ---------------------------------------------------------------- MXFP4 weights


def _mxfp4_golden_tables():
    """{code: Fraction or 'nan'} for e2m1 and e8m0, from tests/golden/mxfp4_decode.txt."""
    e2m1, e8m0 = {}, {}
    for kind, code, value in read_table("mxfp4_decode.txt"):
        v = "nan" if value == "nan" else (exact(value.lstrip("-")) * (-1 if value.startswith("-") else 1),
                                          value.startswith("-"))
        (e2m1 if kind == "e2m1" else e8m0)[int(code)] = v
    return e2m1, e8m0


def check_mxfp4_decode_golden(o):
    e2m1, e8m0 = _mxfp4_golden_tables()
    assert sorted(e2m1) == list(range(16)), "all 16 e2m1 codes are listed"
    for code, (val, neg) in e2m1.items():
        got = o.c.oracle_e2m1_to_f64(code)
        assert Fraction(got) == val and math.copysign(1.0, got) == (-1.0 if neg else 1.0), (code, got)
    for code, v in e8m0.items():
        got = o.c.oracle_e8m0_to_f64(code)
        if v == "nan":
            assert math.isnan(got), (code, got)
        else:
            assert Fraction(got) == v[0], (code, got)


def check_mxfp4_scales_vs_ldexp(o):
    # every finite e8m0 code against the library's power of two
    for s in range(255):
        assert o.c.oracle_e8m0_to_f64(s) == math.ldexp(1.0, s - 127), s
    assert math.isnan(o.c.oracle_e8m0_to_f64(255))


def _mxfp4_golden_projection():
    rows = read_table("mxfp4_projection_worked.txt")
    x_nz = {int(kv.split("=")[0]): exact(kv.split("=")[1]) for kv in rows[0][1:]}
    Ws = [[int(v, 16) for v in r[1:]] for r in rows if r[0] == "Ws:"]
    Wq = [[int(v, 16) for v in r[1:]] for r in rows if r[0] == "Wq:"]
    y = [r[1:] for r in rows if r[0] == "y:"][0]
    A = [r[1:] for r in rows if r[0] == "A:"][0]
    return x_nz, np.array(Wq, dtype=np.uint8), np.array(Ws, dtype=np.uint8), y, A


def check_mxfp4_projection_golden(o):
    x_nz, Wq, Ws, y_txt, A_txt = _mxfp4_golden_projection()
    K = 64
    x = np.zeros((1, K), dtype=np.float32)
    for k, v in x_nz.items():
        x[0, k] = float(v)
    xb = bits_of(x)
    assert np.array_equal(values(xb), x.astype(np.float64)), "x values exact in bf16"
    y, A = o.projection_mxfp4(xb, Wq, Ws)
    for n, (ty, ta) in enumerate(zip(y_txt, A_txt)):
        if ty == "nan":
            assert math.isnan(y[0, n]) and math.isnan(A[0, n]), n
        else:
            assert Fraction(y[0, n]) == exact(ty) and Fraction(A[0, n]) == exact(ta), (n, y[0, n], A[0, n])


def _mxfp4_dequant_bf16(Wq, Ws):
    """Dequantised weights as bf16 bits, built without the oracle: nibbles unpacked with
    numpy (element 2i low, 2i+1 high), values from the golden e2m1 table, scales by
    math.ldexp, rounded to bf16 by torch (exact: at most 2 significant bits)."""
    e2m1, _ = _mxfp4_golden_tables()
    table = np.array([float(e2m1[c][0]) * (-1.0 if e2m1[c][1] and e2m1[c][0] == 0 else 1.0)
                      for c in range(16)])
    N = Wq.shape[0]
    codes = np.stack([Wq & 0x0F, Wq >> 4], axis=-1).reshape(N, -1)
    K = codes.shape[1]
    scale = np.array([[math.ldexp(1.0, int(s) - 127) if s != 255 else math.nan for s in row]
                      for row in Ws])
    w = table[codes] * np.repeat(scale, 32, axis=1)[:, :K]
    wb = bits_of(w.astype(np.float32))
    assert np.array_equal(values(wb), w, equal_nan=True), "dequantised weights exact in bf16"
    return wb


def check_mxfp4_vs_bf16_projection(o):
    # the MXFP4 projection equals the (separately pinned) bf16 projection of the
    # dequantised weights, term for term: the same products in the same order
    rng = np.random.default_rng(31)
    for M, N, K in [(1, 5, 32), (3, 7, 96), (2, 16, 256)]:
        x = random_bf16((M, K), 40 + K)
        Wq = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
        Ws = rng.integers(110, 135, (N, K // 32)).astype(np.uint8)
        y4, A4 = o.projection_mxfp4(x, Wq, Ws)
        y16, A16 = o.projection(x, _mxfp4_dequant_bf16(Wq, Ws))
        assert np.array_equal(y4, y16) and np.array_equal(A4, A16), (M, N, K)


def check_mxfp4_exact_small(o):
    # exact rational brute force over the dequantised weights
    rng = np.random.default_rng(32)
    M, N, K = 2, 3, 64
    x = random_bf16((M, K), 77)
    Wq = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    Ws = rng.integers(118, 132, (N, K // 32)).astype(np.uint8)
    y, A = o.projection_mxfp4(x, Wq, Ws)
    ye, Ae = exact_projection(x, _mxfp4_dequant_bf16(Wq, Ws))
    for m in range(M):
        for n in range(N):
            assert y[m, n] == float(ye[m][n]) and A[m, n] == float(Ae[m][n]), (m, n)


def check_mxfp4_nan_scale_rows(o):
    # a NaN scale poisons exactly the rows that use its block
    rng = np.random.default_rng(33)
    M, N, K = 2, 4, 96
    x = random_bf16((M, K), 5)
    Wq = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    Ws = np.full((N, K // 32), 127, dtype=np.uint8)
    Ws[2, 1] = 255
    y = o.projection_mxfp4(x, Wq, Ws, with_scale=False)
    assert np.isnan(y[:, 2]).all() and not np.isnan(np.delete(y, 2, axis=1)).any()


def _e4m3_golden():
    """{code: (Fraction magnitude, negative) or 'nan'} from tests/golden/fp8_e4m3_decode.txt."""
    out = {}
    for code, value in read_table("fp8_e4m3_decode.txt"):
        out[int(code, 16)] = "nan" if value == "nan" else (exact(value.lstrip("-")),
                                                           value.startswith("-"))
    return out


def check_fp8_decode_golden(o):
    for code, v in _e4m3_golden().items():
        got = o.c.oracle_e4m3_to_f64(code)
        if v == "nan":
            assert math.isnan(got), (code, got)
        else:
            mag, neg = v
            assert Fraction(abs(got)) == mag and math.copysign(1.0, got) == (-1.0 if neg else 1.0), \
                (hex(code), got)


def _torch_e4m3(codes: np.ndarray) -> np.ndarray:
    """torch's float8_e4m3fn conversion of the codes, as float64 (a library routine)."""
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def check_fp8_decode_vs_torch(o):
    codes = np.arange(256, dtype=np.uint8)
    ref = _torch_e4m3(codes)
    got = o.e4m3_to_f64(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok]), "every finite e4m3 code"
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok])), "signed zeros"


def _fp8_weights(N, K, seed, pow2_scales):
    rng = np.random.default_rng(seed)
    Wq = rng.integers(0, 256, (N, K)).astype(np.uint8)
    Wq[(Wq & 0x7F) == 0x7F] = 0x38  # no NaN codes here
    shape = (-(-N // 128), -(-K // 128))
    if pow2_scales:
        Ws = np.ldexp(1.0, rng.integers(-12, 4, shape)).astype(np.float32)
    else:
        Ws = rng.uniform(0.001, 0.05, shape).astype(np.float32)
    return Wq, Ws


def _fp8_dequant(Wq, Ws):
    """Weights in float64 without the oracle: torch's e4m3 conversion times the block
    scale, expanded over 128 x 128 blocks with numpy."""
    N, K = Wq.shape
    scale = np.repeat(np.repeat(Ws.astype(np.float64), 128, axis=0), 128, axis=1)[:N, :K]
    return _torch_e4m3(Wq) * scale


def check_fp8_projection_vs_numpy(o):
    # numpy float64 matmul on the independently dequantised weights; shapes cross the
    # 128-row and 128-column block edges, every block with its own scale
    for M, N, K, seed in [(2, 200, 300, 1), (1, 130, 136, 2), (3, 5, 8, 3), (2, 257, 129, 4)]:
        x = random_bf16((M, K), 60 + seed)
        Wq, Ws = _fp8_weights(N, K, seed, pow2_scales=False)
        y, A = o.projection_fp8(x, Wq, Ws)
        w = _fp8_dequant(Wq, Ws)
        xv = values(x)
        ref, ref_a = xv @ w.T, np.abs(xv) @ np.abs(w).T
        close(y, ref, ref_a, 1e-12, f"fp8 projection {M}x{N}x{K}")
        close(A, ref_a, ref_a, 1e-12, f"fp8 scale {M}x{N}x{K}")


def check_fp8_exact_small(o):
    # exact rational brute force (power-of-two block scales: every double sum exact)
    M, N, K = 2, 3, 40
    x = random_bf16((M, K), 91)
    Wq, Ws = _fp8_weights(N, K, 92, pow2_scales=True)
    y, A = o.projection_fp8(x, Wq, Ws)
    w = _fp8_dequant(Wq, Ws)
    for m in range(M):
        for n in range(N):
            terms = [Fraction(float(values(x[m:m + 1, k:k + 1])[0, 0])) * Fraction(float(w[n, k]))
                     for k in range(K)]
            assert y[m, n] == float(sum(terms)), (m, n)
            assert A[m, n] == float(sum(abs(t) for t in terms)), (m, n)


def check_fp8_nan_code_rows(o):
    # a NaN code poisons exactly its row
    M, N, K = 2, 4, 64
    x = random_bf16((M, K), 7)
    Wq, Ws = _fp8_weights(N, K, 8, pow2_scales=True)
    Wq[1, 5] = 0xFF
    y = o.projection_fp8(x, Wq, Ws, with_scale=False)
    assert np.isnan(y[:, 1]).all() and not np.isnan(np.delete(y, 1, axis=1)).any()


ALL_CHECKS = [
    check_bf16_decode_golden, check_bf16_decode_all_patterns, check_bf16_round_golden,
    check_bf16_round_vs_torch, check_bf16_round_bruteforce,
    check_projection_golden, check_projection_exact_small, check_projection_integer,
    check_projection_vs_numpy, check_projection_layout, check_projection_identity_zero,
    check_projection_linearity, check_projection_rows,
    check_splitk, check_splitk_sum_order, check_residual,
    check_moe_golden, check_moe_bruteforce, check_grouped,
    check_router_topk_golden, check_router_topk_vs_sort,
    check_mxfp4_decode_golden, check_mxfp4_scales_vs_ldexp, check_mxfp4_projection_golden,
    check_mxfp4_vs_bf16_projection, check_mxfp4_exact_small, check_mxfp4_nan_scale_rows,
    check_fp8_decode_golden, check_fp8_decode_vs_torch, check_fp8_projection_vs_numpy,
    check_fp8_exact_small, check_fp8_nan_code_rows,
]


def run_all(o) -> dict:
    """Run every check; map check name -> None (passed) or the failure message."""
    results = {}
    for chk in ALL_CHECKS:
        try:
            chk(o)
            results[chk.__name__] = None
        except Exception as exc:  # noqa: BLE001 - report every failure kind
            results[chk.__name__] = f"{type(exc).__name__}: {exc}"[:300]
    return results


if __name__ == "__main__":
    # Runner used by the mutation tests: python oracle_pins.py <liboracle.so>
    import json
    import sys
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import oracle
    res = run_all(oracle.Oracle(oracle.load(sys.argv[1])))
    print(json.dumps(res))
