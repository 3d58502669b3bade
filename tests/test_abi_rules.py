"""The argument rules of every C-ABI entry point, checked on the CPU against a
model written from the header's contract alone.

Seeded random calls combine shapes (valid, at the limits and invalid), NULL
pointers, misaligned pointers and buffers that overlap. The library under
test is the C-ABI source linked against host-only launch stubs that count
launches (no GPU code runs). The property:
  * a call that breaks no rule returns MOEF_OK and reaches exactly one launch
    (none when its count, num_tokens or n, is 0: a no-op);
  * a call that breaks rules returns the status of one of the rules it breaks
    and launches nothing.
The model accepts any broken rule's status, so it does not assume an order of
checks; where the header allows two statuses for one rule (hidden above the
limit: "out of range" or "too large"), either is accepted. Overlap rules need
valid sizes, so they are only judged on calls with a valid shape."""
import ctypes
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
STUB = os.path.join(ROOT, "tests", "c", "libmoef_host_stub.so")

OK, NULLP, SHAPE, UNSUP, MISAL, FORMAT, ALIAS = 0, 1, 2, 3, 4, 5, 6
ALL = {OK, NULLP, SHAPE, UNSUP, MISAL, FORMAT, ALIAS}
MAX_TOP_K, MAX_HIDDEN, MAX_HIDDEN_RMSNORM, QUANT_BLOCK = 16, 1 << 20, 16384, 128
MAX_GATE_EXPERTS, MAX_EP_PARTIALS, MAX_AR_RANKS = 512, 64, 16
I32 = 2 ** 31 - 1
MAX_UNITS = 2 ** 26 - 4      # one-wave units a launch may hold (MOEF_MAX_UNITS)
MAX_ITEMS = 2 ** 32 - 256    # one-lane items (MOEF_MAX_ITEMS)

vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
ROUTED = [vp, i64, vp, vp, vp, vp, f32]
FUNCS = {
    "plain": ("moe_finalize", ROUTED + [vp, i64, i64, i32, vp, vp]),
    "rmsnorm": ("moe_finalize_residual_rmsnorm",
                ROUTED + [vp, vp, f32, vp, vp, i64, i64, i32, vp, vp]),
    "quant": ("moe_finalize_quant_ue8m0", ROUTED + [vp, vp, i64, i64, i32, vp, vp]),
    "decode": ("moe_topk_packed_decode", [vp, i64, vp, vp, vp]),
    "gate": ("moe_topk_sigmoid_gate", [vp, i64, i32, i32, vp, vp, vp, vp]),
    "aq_ue8m0": ("moe_act_quant_fp8_ue8m0", [vp, i64, i64, vp, vp, vp]),
    "aq_amax": ("moe_act_quant_fp8_amax", [vp, i64, i64, vp, vp, vp]),
    "combine": ("moe_finalize_ep_combine", [vp, i32, vp, vp, i64, i64, vp]),
    "allreduce": ("moe_allreduce_residual_rmsnorm",
                  [ctypes.POINTER(vp), i32, vp, vp, f32, vp, vp, i64, i64, vp]),
}
ROUTED_KINDS = ("plain", "rmsnorm", "quant")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(STUB):
        pytest.fail(f"{STUB} is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(STUB)
    for name, args in FUNCS.values():
        getattr(L, name).argtypes = args
        getattr(L, name).restype = ctypes.c_int
    L.moef_stub_launch_count.restype = ctypes.c_int
    return L


# ----------------------------------------------------- the header's rules

def chunks(H):
    return -(-H // 512)


def shape_rules(kind, c):
    """Statuses of the broken shape rules."""
    v = set()
    if kind in ROUTED_KINDS:
        T, H, k, P = c["T"], c["H"], c["k"], c["P"]
        if T < 0 or P < 0 or not 1 <= k <= MAX_TOP_K or H < 1:
            v.add(SHAPE)
        if H >= 1:
            if H % 8:
                v.add(UNSUP)
            if H > MAX_HIDDEN:
                v |= {SHAPE, UNSUP}
            if P > I32 or T > I32 or (T >= 0 and T * chunks(H) > MAX_UNITS):
                v.add(UNSUP)
            if kind == "rmsnorm" and H > MAX_HIDDEN_RMSNORM:
                v.add(UNSUP)
            if kind == "quant" and H % QUANT_BLOCK:
                v.add(UNSUP)
    elif kind == "decode":
        if c["n"] < 0:
            v.add(SHAPE)
        if c["n"] > MAX_ITEMS:
            v.add(UNSUP)
    elif kind == "gate":
        T, E, k = c["T"], c["E"], c["k"]
        if T < 0 or E < 1 or not 1 <= k <= min(E, MAX_TOP_K):
            v.add(SHAPE)
        if E > MAX_GATE_EXPERTS or T > MAX_UNITS:
            v.add(UNSUP)
    elif kind in ("aq_ue8m0", "aq_amax"):
        T, H = c["T"], c["H"]
        if T < 0 or H < 1:
            v.add(SHAPE)
        if H >= 1 and (H % QUANT_BLOCK or H > MAX_HIDDEN or
                       (T >= 0 and T * chunks(H) > MAX_UNITS)):
            v.add(UNSUP)
    elif kind == "combine":
        T, H, R = c["T"], c["H"], c["R"]
        if T < 0 or H < 1 or not 1 <= R <= MAX_EP_PARTIALS:
            v.add(SHAPE)
        if H >= 1 and (H % 8 or H > MAX_HIDDEN or (T >= 0 and T * (H // 8) > MAX_ITEMS)):
            v.add(UNSUP)
    elif kind == "allreduce":
        T, H, R = c["T"], c["H"], c["R"]
        if T < 0 or H < 1 or not 1 <= R <= MAX_AR_RANKS:
            v.add(SHAPE)
        if H >= 1 and (H % 8 or H > MAX_HIDDEN_RMSNORM or (T >= 0 and T * chunks(H) > MAX_UNITS)):
            v.add(UNSUP)
    return v


def count(kind, c):
    return c["n"] if kind == "decode" else c["T"]


def ranks(c):
    return [f"r{i}" for i in range(max(c["R"], 0))] if 1 <= c["R"] <= MAX_AR_RANKS else []


def layout(kind, c):
    """(alignment by name, inputs, outputs, sizes by name) of a call."""
    T, H = c.get("T", 0), c.get("H", 0)
    if kind in ROUTED_KINDS:
        k, P = c["k"], c["P"]
        align = dict(g2=16, sh=16, idx=4, w32=4, pk=4, err=4)
        size = dict(g2=P * H * 2, idx=T * k * 4, w32=T * k * 4, pk=T * k * 4, sh=T * H * 2, err=4)
        ins = ["g2", "idx", "w32", "pk", "sh"]
        if kind == "plain":
            align.update(out=16)
            size.update(out=T * H * 2)
            outs = ["out"]
        elif kind == "rmsnorm":
            align.update(res=16, gam=16, ro=16, nm=16)
            size.update(res=T * H * 2, gam=H * 2, ro=T * H * 2, nm=T * H * 2)
            ins += ["res", "gam"]
            outs = ["ro", "nm"]
        else:
            align.update(q=8, s=1)
            size.update(q=T * H, s=T * (H // QUANT_BLOCK))
            outs = ["q", "s"]
        return align, ins, outs + ["err"], size
    if kind == "decode":
        n = c["n"]
        return dict(pk=4, ids=4, w=4), ["pk"], ["ids", "w"], dict(pk=n * 4, ids=n * 4, w=n * 4)
    if kind == "gate":
        ob = T * c["k"] * 4
        return (dict(lg=4, ids=4, w=4, pk=4), ["lg"], ["ids", "w", "pk"],
                dict(lg=T * c["E"] * 4, ids=ob, w=ob, pk=ob))
    if kind in ("aq_ue8m0", "aq_amax"):
        sb = T * (H // QUANT_BLOCK) * (4 if kind == "aq_amax" else 1)
        return (dict(x=16, q=8, s=4 if kind == "aq_amax" else 1), ["x"], ["q", "s"],
                dict(x=T * H * 2, q=T * H, s=sb))
    if kind == "combine":
        return (dict(parts=16, sh=16, out=16), ["parts", "sh"], ["out"],
                dict(parts=c["R"] * T * H * 2, sh=T * H * 2, out=T * H * 2))
    rs = ranks(c)
    align = dict(res=16, gam=16, ro=16, nm=16, **{r: 16 for r in rs})
    size = dict(res=T * H * 2, gam=H * 2, ro=T * H * 2, nm=T * H * 2, **{r: T * H * 2 for r in rs})
    return align, rs + ["res", "gam"], ["ro", "nm"], size


def required(kind, c):
    """Names that must not be NULL, and a list of groups of which at least
    one member must be non-NULL."""
    if kind in ROUTED_KINDS:
        names = ["idx"] + (["g2"] if c["P"] > 0 else []) + {
            "plain": ["out"], "rmsnorm": ["res", "gam", "ro", "nm"], "quant": ["q", "s"]}[kind]
        return names, []
    if kind == "decode":
        return ["pk"], [["ids", "w"]]
    if kind == "gate":
        return ["lg", "ids"], []
    if kind in ("aq_ue8m0", "aq_amax"):
        return ["x", "q", "s"], []
    if kind == "combine":
        return ["parts", "out"], []
    return ranks(c) + ["res", "gam", "ro", "nm"], []


def overlap(a, n, b, m):
    return a != 0 and b != 0 and n > 0 and m > 0 and a < b + m and b < a + n


def pointer_rules(kind, c, with_alias):
    v = set()
    if kind in ROUTED_KINDS and (c["w32"] == 0) == (c["pk"] == 0):
        v.add(FORMAT)
    names, groups = required(kind, c)
    if any(c[n] == 0 for n in names) or any(all(c[n] == 0 for n in g) for g in groups):
        v.add(NULLP)
    if kind == "allreduce" and c["arr_null"]:
        v.add(NULLP)
    align, ins, outs, size = layout(kind, c)
    if any(c[n] % a for n, a in align.items() if c.get(n)):
        v.add(MISAL)
    if with_alias:
        for o in outs:
            for i in ins:
                if o == "ro" and i == "res" and c["ro"] == c["res"]:
                    continue                     # the in-place residual update
                if overlap(c[o], size[o], c[i], size[i]):
                    v.add(ALIAS)
        for x, o in enumerate(outs):
            for p in outs[x + 1:]:
                if overlap(c[o], size[o], c[p], size[p]):
                    v.add(ALIAS)
    return v


def expected(kind, c):
    """(set of acceptable statuses, launches expected)."""
    v = shape_rules(kind, c)
    if count(kind, c) == 0:
        return (v or {OK}), 0
    if v:
        return v | pointer_rules(kind, c, with_alias=False), 0
    v = pointer_rules(kind, c, with_alias=True)
    return (v, 0) if v else ({OK}, 1)


# ---------------------------------------------------------- random calls

REGION = 1 << 40          # each buffer starts in its own 1 TiB region


def draw_count(rng, small=300):
    r = rng.random()
    if r < 0.05:
        return 0
    if r < 0.08:
        return int(rng.choice([-1, -5]))
    if r < 0.11:
        return int(rng.choice([I32 - 4, I32 - 3, I32, I32 + 1, 1 << 30, 1 << 21, MAX_UNITS,
                               MAX_UNITS + 1, MAX_UNITS // 14, MAX_UNITS // 14 + 1]))
    return int(rng.integers(1, small))


def draw_hidden(rng, step, top=16384, bad=(0, -8, 4, 1001, 1000, 16392, 1 << 20,
                                            (1 << 20) + 8, 1 << 21, 136)):
    if rng.random() < 0.12:
        return int(rng.choice(bad))
    return step * int(rng.integers(1, top // step + 1))


# pointers a call may leave NULL (the routed err_flag is drawn on its own)
OPTIONAL = dict(plain=["sh"], rmsnorm=["sh"], quant=["sh"], decode=["ids", "w"], gate=["w", "pk"],
                combine=["sh"])


def draw(rng, kind):
    c = {}
    if kind in ROUTED_KINDS:
        c["T"] = draw_count(rng)
        c["H"] = draw_hidden(rng, QUANT_BLOCK if kind == "quant" else 8)
        c["k"] = int(rng.integers(1, 17)) if rng.random() > 0.08 else int(
            rng.choice([0, -1, 17, 100]))
        c["P"] = int(rng.integers(1, 100_000))
        if rng.random() < 0.05:
            c["P"] = 0
        elif rng.random() < 0.04:
            c["P"] = int(rng.choice([-1, I32, I32 + 1]))
        names = ["g2", "idx", "w32", "pk", "sh", "err"] + {
            "plain": ["out"], "rmsnorm": ["res", "gam", "ro", "nm"], "quant": ["q", "s"]}[kind]
    elif kind == "decode":
        c["n"] = draw_count(rng, 5000)
        if rng.random() < 0.03:
            c["n"] = int(rng.choice([I32 * 256, I32 * 256 + 1, MAX_ITEMS, MAX_ITEMS + 1]))
        names = ["pk", "ids", "w"]
    elif kind == "gate":
        c["T"] = draw_count(rng)
        c["E"] = int(rng.integers(1, 513)) if rng.random() > 0.08 else int(
            rng.choice([0, -1, 513, 1024]))
        c["k"] = int(rng.integers(1, min(max(c["E"], 1), 16) + 1)) if rng.random() > 0.1 else int(
            rng.choice([0, -1, 17, c["E"] + 1]))
        names = ["lg", "ids", "w", "pk"]
    elif kind in ("aq_ue8m0", "aq_amax"):
        c["T"] = draw_count(rng)
        c["H"] = draw_hidden(rng, QUANT_BLOCK)
        names = ["x", "q", "s"]
    elif kind == "combine":
        c["T"] = draw_count(rng)
        c["H"] = draw_hidden(rng, 8)
        c["R"] = int(rng.integers(1, 9)) if rng.random() > 0.08 else int(
            rng.choice([0, -1, 64, 65]))
        if c["T"] > 0 and c["H"] > 0 and rng.random() < 0.03:
            c["T"] = MAX_ITEMS // (c["H"] // 8 or 1) + int(rng.integers(0, 2))
        names = ["parts", "sh", "out"]
    else:
        c["T"] = draw_count(rng)
        c["H"] = draw_hidden(rng, 8)
        c["R"] = int(rng.integers(1, 17)) if rng.random() > 0.08 else int(
            rng.choice([0, -1, 17, 20]))
        c["arr_null"] = rng.random() < 0.03
        names = [f"r{i}" for i in range(max(c["R"], 1))] + ["res", "gam", "ro", "nm"]
    c["names"] = names
    for n, name in enumerate(names):
        c[name] = (n + 1) * REGION + 4096 * int(rng.integers(0, 1024))
    if kind in ROUTED_KINDS:
        f = rng.random()
        if f < 0.05:
            pass
        elif f < 0.10:
            c["w32"] = c["pk"] = 0
        elif f < 0.55:
            c["pk"] = 0
        else:
            c["w32"] = 0
        if rng.random() < 0.5:
            c["err"] = 0
    for opt in OPTIONAL.get(kind, ()):
        if rng.random() < 0.3:
            c[opt] = 0
    if kind in ("rmsnorm", "allreduce") and rng.random() < 0.2:
        c["ro"] = c["res"]                               # in place
    for name in names:
        if c[name] and rng.random() < 0.03:
            c[name] = 0
        if c[name] and rng.random() < 0.03:
            c[name] += int(rng.choice([1, 2, 4, 8]))
    if rng.random() < 0.25:                              # one output inside another buffer
        valid = {k: max(v, 0) for k, v in c.items() if isinstance(v, int) and k in
                 ("T", "H", "k", "P", "n", "E", "R")}
        _, _, outs, size = layout(kind, dict(c, **valid))
        outs = [o for o in outs if c.get(o)]
        o = str(rng.choice(outs)) if outs else None
        others = [n for n in names if n != o and c[n] and n in size]
        if o is not None and others:
            t = str(rng.choice(others))
            span = size[t]
            c[o] = c[t] + (16 * int(rng.integers(0, max(1, span // 16))) if span > 0 else 0)
    return c


def call(L, kind, c):
    name, _ = FUNCS[kind]
    p = lambda n: c[n] or None                            # noqa: E731
    if kind in ROUTED_KINDS:
        args = [p("g2"), c["P"], p("idx"), p("w32"), p("pk"), p("sh"), 2.5]
        if kind == "plain":
            args += [p("out"), c["T"], c["H"], c["k"], p("err"), None]
        elif kind == "rmsnorm":
            args += [p("res"), p("gam"), 1e-6, p("ro"), p("nm"), c["T"], c["H"], c["k"], p("err"),
                     None]
        else:
            args += [p("q"), p("s"), c["T"], c["H"], c["k"], p("err"), None]
    elif kind == "decode":
        args = [p("pk"), c["n"], p("ids"), p("w"), None]
    elif kind == "gate":
        args = [p("lg"), c["T"], c["E"], c["k"], p("ids"), p("w"), p("pk"), None]
    elif kind in ("aq_ue8m0", "aq_amax"):
        args = [p("x"), c["T"], c["H"], p("q"), p("s"), None]
    elif kind == "combine":
        args = [p("parts"), c["R"], p("sh"), p("out"), c["T"], c["H"], None]
    else:
        rank_names = [f"r{i}" for i in range(max(c["R"], 1))]
        arr = None if c["arr_null"] else (vp * len(rank_names))(*[p(r) for r in rank_names])
        args = [arr, c["R"], p("res"), p("gam"), 1e-6, p("ro"), p("nm"), c["T"], c["H"], None]
    before = L.moef_stub_launch_count()
    st = getattr(L, name)(*args)
    return st, L.moef_stub_launch_count() - before


@pytest.mark.parametrize("kind", list(FUNCS))
def test_random_calls_follow_the_header_rules(lib, kind):
    rng = np.random.default_rng(list(FUNCS).index(kind) + 11)
    seen = set()
    for i in range(6000 if kind in ROUTED_KINDS else 3000):
        c = draw(rng, kind)
        want, launches = expected(kind, c)
        st, n = call(lib, kind, c)
        assert st in want and n == launches, (
            f"call {i}: status {st}, launches {n}; the rules allow {sorted(want)} with "
            f"{launches} launch(es); arguments { {k: v for k, v in c.items() if k != 'names'} }")
        seen.add(st)
    # the draw reaches every outcome the entry point has
    reachable = ALL if kind in ROUTED_KINDS else ALL - {FORMAT}
    assert seen == reachable, seen


def test_model_examples():
    """The model itself on hand-made cases (so a slip in it cannot hide a
    library bug behind a matching slip)."""
    R40 = 1 << 40
    base = dict(T=4, H=1024, k=8, P=64, g2=R40, idx=2 * R40, w32=3 * R40, pk=0, sh=0, err=0,
                out=4 * R40)
    assert expected("plain", base) == ({OK}, 1)
    assert expected("plain", dict(base, T=0, g2=0, idx=0, out=0)) == ({OK}, 0)
    assert expected("plain", dict(base, k=17))[0] == {SHAPE}
    assert expected("plain", dict(base, H=1028))[0] == {UNSUP}
    assert expected("plain", dict(base, H=(1 << 20) + 8))[0] == {SHAPE, UNSUP}
    assert expected("plain", dict(base, pk=5 * R40))[0] == {FORMAT}
    assert expected("plain", dict(base, w32=0))[0] == {FORMAT}
    assert expected("plain", dict(base, out=R40 + 64 * 2048 - 16))[0] == {ALIAS}
    assert expected("plain", dict(base, out=R40 + 64 * 2048))[0] == {OK}
    assert expected("plain", dict(base, err=4 * R40 + 4 * 1024 * 2 - 4))[0] == {ALIAS}
    assert expected("plain", dict(base, out=4 * R40 + 8))[0] == {MISAL}
    assert expected("plain", dict(base, g2=0, P=0)) == ({OK}, 1)
    assert expected("plain", dict(base, g2=0))[0] == {NULLP}
    assert expected("plain", dict(base, P=I32 + 1))[0] == {UNSUP}
    r = {k: v for k, v in base.items() if k != "out"}
    r.update(res=5 * R40, gam=6 * R40, ro=5 * R40, nm=7 * R40)
    assert expected("rmsnorm", r) == ({OK}, 1)
    assert expected("rmsnorm", dict(r, ro=5 * R40 + 16))[0] == {ALIAS}
    assert expected("rmsnorm", dict(r, nm=5 * R40))[0] == {ALIAS}
    assert expected("rmsnorm", dict(r, H=16392))[0] == {UNSUP}
    q = {k: v for k, v in base.items() if k != "out"}
    q.update(q=5 * R40, s=5 * R40 + 4 * 1024)
    assert expected("quant", q) == ({OK}, 1)
    assert expected("quant", dict(q, s=5 * R40 + 4 * 1024 - 1))[0] == {ALIAS}
    assert expected("quant", dict(q, H=1000))[0] == {UNSUP}
    d = dict(n=10, pk=R40, ids=2 * R40, w=0)
    assert expected("decode", d) == ({OK}, 1)
    assert expected("decode", dict(d, ids=0))[0] == {NULLP}
    assert expected("decode", dict(d, ids=R40 + 36))[0] == {ALIAS}
    assert expected("decode", dict(d, ids=R40 + 40)) == ({OK}, 1)
    assert expected("decode", dict(d, n=-1))[0] == {SHAPE}
    g = dict(T=3, E=256, k=8, lg=R40, ids=2 * R40, w=0, pk=3 * R40 + 2)
    assert expected("gate", g)[0] == {MISAL}
    assert expected("gate", dict(g, pk=0)) == ({OK}, 1)
    assert expected("gate", dict(g, k=9, E=8, pk=0))[0] == {SHAPE}
    assert expected("gate", dict(g, E=513, pk=0))[0] == {UNSUP}
    a = dict(T=2, H=256, x=R40, q=2 * R40, s=2 * R40 + 512)
    assert expected("aq_ue8m0", a) == ({OK}, 1)
    assert expected("aq_amax", a) == ({OK}, 1)
    assert expected("aq_amax", dict(a, s=2 * R40 + 504))[0] == {ALIAS}       # codes' last 8 B
    assert expected("aq_amax", dict(a, s=2 * R40 + 514))[0] == {MISAL}       # 4-byte rule
    assert expected("aq_ue8m0", dict(a, s=2 * R40 + 514)) == ({OK}, 1)       # bytes: no rule
    assert expected("aq_ue8m0", dict(a, s=0, H=100))[0] == {UNSUP, NULLP}
    cb = dict(T=2, H=64, R=3, parts=R40, sh=0, out=R40 + 3 * 2 * 64 * 2)
    assert expected("combine", cb) == ({OK}, 1)
    assert expected("combine", dict(cb, out=R40 + 3 * 2 * 64 * 2 - 16))[0] == {ALIAS}
    ar = dict(T=2, H=64, R=2, arr_null=False, r0=R40, r1=2 * R40, res=3 * R40, gam=4 * R40,
              ro=3 * R40, nm=5 * R40)
    assert expected("allreduce", ar) == ({OK}, 1)
    assert expected("allreduce", dict(ar, arr_null=True))[0] == {NULLP}
    assert expected("allreduce", dict(ar, ro=2 * R40))[0] == {ALIAS}
    assert expected("allreduce", dict(ar, R=17))[0] == {SHAPE}
