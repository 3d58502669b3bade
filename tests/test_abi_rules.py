"""The argument rules of the three routed entry points (moe_finalize,
moe_finalize_residual_rmsnorm, moe_finalize_quant_ue8m0), checked on the CPU
against a model written from the header's contract alone.

Seeded random calls combine shapes (valid, at the limits and invalid), NULL
pointers, misaligned pointers and buffers that overlap. The library under
test is the C-ABI source linked against host-only launch stubs that count
launches (no GPU code runs). The property:
  * a call that breaks no rule returns MOEF_OK and reaches exactly one launch
    (none when num_tokens is 0, a no-op);
  * a call that breaks rules returns the status of one of the rules it breaks
    and launches nothing.
The model accepts any broken rule's status, so it does not assume an order of
checks; where the header allows two statuses for one rule (hidden above the
limit: "out of range" or "too large"), either is accepted."""
import ctypes
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
STUB = os.path.join(ROOT, "tests", "c", "libmoef_host_stub.so")

OK, NULLP, SHAPE, UNSUP, MISAL, FORMAT, ALIAS = 0, 1, 2, 3, 4, 5, 6
MAX_TOP_K, MAX_HIDDEN, MAX_HIDDEN_RMSNORM, QUANT_BLOCK = 16, 1 << 20, 16384, 128
I32 = 2 ** 31 - 1

vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
ROUTED = [vp, i64, vp, vp, vp, vp, f32]
SIGNATURES = {
    "plain": ("moe_finalize", ROUTED + [vp, i64, i64, i32, vp, vp]),
    "rmsnorm": ("moe_finalize_residual_rmsnorm",
                ROUTED + [vp, vp, f32, vp, vp, i64, i64, i32, vp, vp]),
    "quant": ("moe_finalize_quant_ue8m0", ROUTED + [vp, vp, i64, i64, i32, vp, vp]),
}


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(STUB):
        pytest.fail(f"{STUB} is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(STUB)
    for name, args in SIGNATURES.values():
        getattr(L, name).argtypes = args
        getattr(L, name).restype = ctypes.c_int
    L.moef_stub_launch_count.restype = ctypes.c_int
    return L


# ----------------------------------------------------- the header's rules

def shape_rules(kind, T, H, k, P):
    """Statuses of the broken shape rules."""
    v = set()
    if T < 0 or P < 0 or not 1 <= k <= MAX_TOP_K or H < 1:
        v.add(SHAPE)
    if H >= 1:
        if H % 8:
            v.add(UNSUP)
        if H > MAX_HIDDEN:
            v |= {SHAPE, UNSUP}
        if P > I32 or T > I32 or (T >= 0 and T * -(-H // 512) > I32):
            v.add(UNSUP)
        if kind == "rmsnorm" and H > MAX_HIDDEN_RMSNORM:
            v.add(UNSUP)
        if kind == "quant" and H % QUANT_BLOCK:
            v.add(UNSUP)
    return v


def overlap(a, n, b, m):
    return a != 0 and b != 0 and n > 0 and m > 0 and a < b + m and b < a + n


def pointer_rules(kind, c):
    """Statuses of the broken pointer rules of a call with a valid shape and
    num_tokens >= 1: formats, NULLs, alignment, aliasing."""
    T, H, k, P = c["T"], c["H"], c["k"], c["P"]
    v = set()
    if (c["w32"] == 0) == (c["pk"] == 0):
        v.add(FORMAT)
    if c["idx"] == 0 or (c["g2"] == 0 and P > 0):
        v.add(NULLP)
    outs = {"plain": ["out"], "rmsnorm": ["ro", "nm"], "quant": ["q", "s"]}[kind]
    required = outs + (["res", "gam"] if kind == "rmsnorm" else [])
    if any(c[n] == 0 for n in required):
        v.add(NULLP)
    align = {"g2": 16, "sh": 16, "idx": 4, "w32": 4, "pk": 4, "err": 4, "out": 16, "res": 16,
             "gam": 16, "ro": 16, "nm": 16, "q": 8, "s": 1}
    if any(c[n] % align[n] for n in align if n in c and c[n]):
        v.add(MISAL)
    size = {"g2": P * H * 2, "idx": T * k * 4, "w32": T * k * 4, "pk": T * k * 4,
            "sh": T * H * 2, "res": T * H * 2, "gam": H * 2, "out": T * H * 2, "ro": T * H * 2,
            "nm": T * H * 2, "q": T * H, "s": T * (H // QUANT_BLOCK), "err": 4}
    inputs = ["g2", "idx", "w32", "pk", "sh"] + (["res", "gam"] if kind == "rmsnorm" else [])
    written = outs + ["err"]
    for o in written:
        for i in inputs:
            if o == "ro" and i == "res" and c["ro"] == c["res"]:
                continue                         # the in-place residual update
            if overlap(c[o], size[o], c[i], size[i]):
                v.add(ALIAS)
    for x, o in enumerate(written):
        for p in written[x + 1:]:
            if overlap(c[o], size[o], c[p], size[p]):
                v.add(ALIAS)
    return v, size


def expected(kind, c):
    """(set of acceptable statuses, launches expected)."""
    v = shape_rules(kind, c["T"], c["H"], c["k"], c["P"])
    if v:
        return v, 0
    if c["T"] == 0:
        return {OK}, 0
    v, _ = pointer_rules(kind, c)
    return (v, 0) if v else ({OK}, 1)


# ---------------------------------------------------------- random calls

REGION = 1 << 40          # each buffer starts in its own 1 TiB region


def draw(rng, kind):
    r = rng.random
    T = int(rng.integers(1, 300))
    if r() < 0.05:
        T = 0
    elif r() < 0.03:
        T = int(rng.choice([-1, -5]))
    elif r() < 0.03:
        T = int(rng.choice([I32, I32 + 1, 1 << 30, 1 << 21]))
    step = QUANT_BLOCK if kind == "quant" else 8
    H = step * int(rng.integers(1, 16384 // step + 1))
    if r() < 0.12:
        H = int(rng.choice([0, -8, 4, 1001, 1000, 16392, 1 << 20, (1 << 20) + 8, 1 << 21, 136]))
    k = int(rng.integers(1, 17))
    if r() < 0.08:
        k = int(rng.choice([0, -1, 17, 100]))
    P = int(rng.integers(1, 100_000))
    if r() < 0.05:
        P = 0
    elif r() < 0.04:
        P = int(rng.choice([-1, I32, I32 + 1]))
    names = ["g2", "idx", "w32", "pk", "sh", "err"] + {
        "plain": ["out"], "rmsnorm": ["res", "gam", "ro", "nm"], "quant": ["q", "s"]}[kind]
    c = dict(T=T, H=H, k=k, P=P)
    for n, name in enumerate(names):
        c[name] = (n + 1) * REGION + 4096 * int(rng.integers(0, 1024))
    # routing format: one of the two, sometimes both or neither
    f = r()
    if f < 0.05:
        pass
    elif f < 0.10:
        c["w32"] = c["pk"] = 0
    elif f < 0.55:
        c["pk"] = 0
    else:
        c["w32"] = 0
    if r() < 0.3:
        c["sh"] = 0
    if r() < 0.5:
        c["err"] = 0
    if kind == "rmsnorm" and r() < 0.2:
        c["ro"] = c["res"]                               # in place
    for name in names:
        if c[name] and r() < 0.03:
            c[name] = 0
        if c[name] and r() < 0.03:
            c[name] += int(rng.choice([1, 2, 4, 8]))
    if r() < 0.25:                                       # one output inside another buffer
        outs = [n for n in names if n in ("out", "ro", "nm", "q", "s", "err") and c[n]]
        o = str(rng.choice(outs)) if outs else None
        others = [n for n in names if n != o and c[n]]
        if o is not None and others:
            t = str(rng.choice(others))
            _, size = pointer_rules(kind, dict(c, T=max(T, 0), P=max(P, 0), H=max(H, 0),
                                               k=max(k, 0)))
            span = size[t]
            c[o] = c[t] + (16 * int(rng.integers(0, max(1, span // 16))) if span > 0 else 0)
    return c


def call(L, kind, c):
    name, _ = SIGNATURES[kind]
    p = lambda n: c[n] or None                            # noqa: E731
    head = (p("g2"), c["P"], p("idx"), p("w32"), p("pk"), p("sh"), 2.5)
    if kind == "plain":
        tail = (p("out"), c["T"], c["H"], c["k"], p("err"), None)
    elif kind == "rmsnorm":
        tail = (p("res"), p("gam"), 1e-6, p("ro"), p("nm"), c["T"], c["H"], c["k"], p("err"), None)
    else:
        tail = (p("q"), p("s"), c["T"], c["H"], c["k"], p("err"), None)
    before = L.moef_stub_launch_count()
    st = getattr(L, name)(*head, *tail)
    return st, L.moef_stub_launch_count() - before


@pytest.mark.parametrize("kind", ["plain", "rmsnorm", "quant"])
def test_random_calls_follow_the_header_rules(lib, kind):
    rng = np.random.default_rng({"plain": 11, "rmsnorm": 12, "quant": 13}[kind])
    seen = set()
    for i in range(6000):
        c = draw(rng, kind)
        want, launches = expected(kind, c)
        st, n = call(lib, kind, c)
        assert st in want and n == launches, (
            f"call {i}: status {st}, launches {n}; the rules allow {sorted(want)} with "
            f"{launches} launch(es); arguments {c}")
        seen.add(st)
    # the draw reaches every outcome
    assert seen == {OK, NULLP, SHAPE, UNSUP, MISAL, FORMAT, ALIAS}, seen


def test_model_examples():
    """The model itself on hand-made cases (so a slip in it cannot hide a
    library bug behind a matching slip)."""
    base = dict(T=4, H=1024, k=8, P=64, g2=1 << 40, idx=2 << 40, w32=3 << 40, pk=0, sh=0,
                err=0, out=4 << 40)
    assert expected("plain", base) == ({OK}, 1)
    assert expected("plain", dict(base, T=0, g2=0, idx=0, out=0)) == ({OK}, 0)
    assert expected("plain", dict(base, k=17))[0] == {SHAPE}
    assert expected("plain", dict(base, H=1028))[0] == {UNSUP}
    assert expected("plain", dict(base, H=(1 << 20) + 8))[0] == {SHAPE, UNSUP}
    assert expected("plain", dict(base, pk=5 << 40))[0] == {FORMAT}
    assert expected("plain", dict(base, w32=0))[0] == {FORMAT}
    assert expected("plain", dict(base, out=(1 << 40) + 64 * 2048 - 16))[0] == {ALIAS}
    assert expected("plain", dict(base, out=(1 << 40) + 64 * 2048))[0] == {OK}
    assert expected("plain", dict(base, err=(4 << 40) + 4 * 1024 * 2 - 4))[0] == {ALIAS}
    assert expected("plain", dict(base, out=(4 << 40) + 8))[0] == {MISAL}
    assert expected("plain", dict(base, g2=0, P=0)) == ({OK}, 1)
    assert expected("plain", dict(base, g2=0))[0] == {NULLP}
    assert expected("plain", dict(base, P=I32 + 1))[0] == {UNSUP}
    r = dict(base, out=0, res=5 << 40, gam=6 << 40, ro=5 << 40, nm=7 << 40)
    del r["out"]
    assert expected("rmsnorm", r) == ({OK}, 1)
    assert expected("rmsnorm", dict(r, ro=(5 << 40) + 16))[0] == {ALIAS}
    assert expected("rmsnorm", dict(r, nm=5 << 40))[0] == {ALIAS}
    assert expected("rmsnorm", dict(r, H=16392))[0] == {UNSUP}
    q = dict(base, q=5 << 40, s=(5 << 40) + 4 * 1024)
    del q["out"]
    assert expected("quant", q) == ({OK}, 1)
    assert expected("quant", dict(q, s=(5 << 40) + 4 * 1024 - 1))[0] == {ALIAS}
    assert expected("quant", dict(q, H=1000))[0] == {UNSUP}
