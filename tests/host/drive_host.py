"""Drives a host-only build of libfdec (api.cpp, plan.cpp, tests/host/stubs.cpp),
made with AddressSanitizer and UndefinedBehaviorSanitizer, through every entry
point over seeded random shapes. Run by tests/test_host_sanitizers.py in a child
process (the sanitizer runtime is preloaded there); ctypes and numpy only.

"Device" buffers are host memory that nothing dereferences; each is registered
with the stand-in launchers, which abort when a launch would touch a range
outside them, write overlapping workspace ranges, or write the fused path's
counters from any launch but a fused one. The struct layouts mirror
include/fdec.h.

    python drive_host.py <lib> <cases>
"""
import ctypes
import sys

import numpy as np

P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3


class KV(ctypes.Structure):
    _fields_ = [("k", P), ("v", P), ("dtype", I), ("num_kv_heads", I), ("head_dim", I), ("page_size", I),
                ("capacity", I), ("s_outer", ctypes.c_int64), ("s_token", ctypes.c_int64),
                ("s_head", ctypes.c_int64), ("page_table", P), ("max_pages_per_seq", I), ("k_descale", P),
                ("v_descale", P), ("cache_batch_idx", P), ("cache_leftpad", P)]


class Append(ctypes.Structure):
    _fields_ = [("k_new", P), ("v_new", P), ("rope_cos", P), ("rope_sin", P), ("rotary_dim", I),
                ("rope_max_pos", I)]


lib = ctypes.CDLL(sys.argv[1])
NCASES = int(sys.argv[2]) if len(sys.argv) > 2 else 400
lib.fdec_stub_region.argtypes = [P, Z, ctypes.c_char_p]
lib.fdec_stub_reserve.argtypes = [P, Z]
lib.fdec_last_error.restype = ctypes.c_char_p
for name in ("fdec_workspace_size", "fdec_balanced_workspace_size"):
    getattr(lib, name).restype = Z
    getattr(lib, name).argtypes = [I, I, I, I, I]
lib.fdec_cascade_workspace_size.restype = Z
lib.fdec_cascade_workspace_size.argtypes = [I, I, I, I, I, I]
lib.fdec_split_chunk.restype = ctypes.c_int64
lib.fdec_split_chunk.argtypes = [I, I]
lib.fdec_plan_kv.argtypes = [I, I, I, P, I, I, I, I, ctypes.POINTER(I)]
lib.fdec_plan.argtypes = [I, I, I, P, I, I, I, ctypes.POINTER(I)]
lib.fdec_plan_rules.argtypes = [I, I, I, I, ctypes.POINTER(I)]
lib.fdec_cascade_plan.argtypes = [I, I, I, I, I, I, I, ctypes.POINTER(I), ctypes.POINTER(I)]
lib.fdec_decode.argtypes = [P, I, I, ctypes.POINTER(KV), P, I, F, ctypes.POINTER(Append), I, P, P, P, Z, P]
lib.fdec_decode_partials.argtypes = [P, I, I, ctypes.POINTER(KV), P, I, F, ctypes.POINTER(Append), P, P, P, P]
lib.fdec_merge_states.argtypes = [P, P, P, I, I, I, I, P, P, P]
lib.fdec_decode_balanced.argtypes = [P, I, I, ctypes.POINTER(KV), P, I, F, P, P, P, Z, P]
lib.fdec_decode_multi.argtypes = [P, I, I, I, ctypes.POINTER(KV), P, I, F, P, P, P, Z, P]
lib.fdec_decode_multi_balanced.argtypes = [P, I, I, I, ctypes.POINTER(KV), P, I, F, P, P, P, Z, P]
lib.fdec_cascade_decode.argtypes = [P, I, I, ctypes.POINTER(KV), P, I, P, I, I, F, P, P, P, Z, P]
lib.fdec_trace_start.argtypes = [I]
lib.fdec_trace_stop.argtypes = [P, P, I, ctypes.POINTER(I)]

_keep = []


def buf(nbytes, name):
    """A registered 256-byte aligned "device" buffer of nbytes (at least 256)."""
    n = max(int(nbytes), 256)
    a = np.zeros(n + 512, dtype=np.uint8)
    _keep.append(a)
    addr = (a.ctypes.data + 255) // 256 * 256
    lib.fdec_stub_region(addr, n, name.encode())
    return addr


def check(rc, allowed, what):
    if rc not in allowed:
        raise SystemExit(f"{what}: status {rc} ({lib.fdec_last_error().decode()}), expected one of {allowed}")


def make_kv(rng, B, Hkv, D, dtype, paged):
    es = 1 if dtype == 2 else 2
    kv = KV()
    kv.dtype, kv.num_kv_heads, kv.head_dim = dtype, Hkv, D
    if paged:
        ps = int(rng.choice([16, 32, 64, 256]))
        maxp = int(rng.integers(1, 40))
        pool = int(rng.integers(1, 64))
        kv.page_size, kv.max_pages_per_seq, kv.capacity = ps, maxp, 0
        kv.s_outer, kv.s_token, kv.s_head = ps * Hkv * D, Hkv * D, D
        kv.k = buf(pool * ps * Hkv * D * es, "k")
        kv.v = buf(pool * ps * Hkv * D * es, "v")
        kv.page_table = buf(B * maxp * 4, "page_table")
        cap = ps * maxp
    else:
        cap = int(rng.integers(1, 5000))
        kv.page_size, kv.capacity = 0, cap
        kv.s_outer, kv.s_token, kv.s_head = cap * Hkv * D, Hkv * D, D
        rows = B + int(rng.integers(0, 3))
        kv.k = buf(rows * cap * Hkv * D * es, "k")
        kv.v = buf(rows * cap * Hkv * D * es, "v")
        if rng.random() < 0.3:
            kv.cache_batch_idx = buf(B * 4, "batch_idx")
    if rng.random() < 0.3:
        kv.cache_leftpad = buf(B * 4, "leftpad")
    if dtype == 2 and rng.random() < 0.7:
        kv.k_descale = buf(B * Hkv * 4, "k_descale")
        kv.v_descale = buf(B * Hkv * 4, "v_descale")
    return kv, cap


def plan_splits(B, Hq, kv, cap, S):
    if S > 0:
        return S
    out = I(0)
    check(lib.fdec_plan_kv(B, Hq, kv.num_kv_heads, None, cap, kv.page_size, kv.dtype, 256, ctypes.byref(out)),
          (OK,), "fdec_plan_kv")
    return out.value


def one_case(rng, i):
    B = int(rng.integers(0, 40))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8]))
    Hq = G * Hkv
    D = int(rng.choice([128, 128, 64]))
    dtype = int(rng.choice([0, 1, 2]))
    paged = bool(rng.random() < 0.5)
    lib.fdec_stub_reset()
    kv, cap = make_kv(rng, B, Hkv, D, dtype, paged)
    q_len = int(rng.choice([1, 1, 2, 3, 4, 8, 16]))
    qb = buf(B * q_len * Hq * D * 2, "q")
    lens = buf(B * 4, "seq_lens")
    out = buf(B * q_len * Hq * D * 4, "out")
    lse = buf(B * q_len * Hq * 4, "lse") if rng.random() < 0.8 else None
    kind = rng.choice(["decode", "decode", "fused", "append", "partials", "balanced", "multi", "multi_balanced",
                       "cascade", "noargs"])
    S = int(rng.choice([0, 1, 2, 5, 16, 64, 128, 256]))
    what = f"case {i} {kind} B={B} Hq={Hq} Hkv={Hkv} D={D} dtype={dtype} paged={paged} S={S} q_len={q_len}"
    if kind in ("decode", "fused", "append"):
        Su = plan_splits(B, Hq, kv, cap, S)
        n = lib.fdec_workspace_size(B, Hq, Hkv, D, Su)
        ws = buf(n, "workspace")
        lib.fdec_stub_reserve(ws, B * Hkv * 4)
        app = None
        if kind == "append":
            app = Append()
            app.k_new, app.v_new = buf(B * Hkv * D * 2, "k_new"), buf(B * Hkv * D * 2, "v_new")
            app.rotary_dim = int(rng.choice([0, 64, D]))
            if app.rotary_dim:
                app.rope_max_pos = 4096
                app.rope_cos = buf(4096 * app.rotary_dim // 2 * 4, "cos")
                app.rope_sin = buf(4096 * app.rotary_dim // 2 * 4, "sin")
        rc = lib.fdec_decode(qb, B, Hq, ctypes.byref(kv), lens, S, 0.0, ctypes.byref(app) if app else None,
                             int(kind == "fused"), out, lse, ws, n, None)
        check(rc, (OK,), what)
        if B > 0 and rc == OK:  # one byte less of workspace is refused
            check(lib.fdec_decode(qb, B, Hq, ctypes.byref(kv), lens, S, 0.0, ctypes.byref(app) if app else None,
                                  int(kind == "fused"), out, lse, ws, n - 1, None), (WORKSPACE,), what + " (short)")
    elif kind == "partials":
        Su = max(S, 1)
        rows = B * Hq * Su
        pm, pd, po = buf(rows * 4, "pm"), buf(rows * 4, "pd"), buf(rows * D * 4, "po")
        check(lib.fdec_decode_partials(qb, B, Hq, ctypes.byref(kv), lens, Su, 0.0, None, po, pm, pd, None),
              (OK,), what)
        check(lib.fdec_merge_states(po, pm, pd, B, Hq, Su, D, out, lse, None), (OK,), what + " (merge)")
    elif kind in ("balanced", "multi_balanced"):
        nb = int(rng.choice([0, 1, 3, 64, 256]))
        ql = q_len if kind == "multi_balanced" else 1
        n = lib.fdec_balanced_workspace_size(B, ql * Hq, Hkv, D, nb)
        ws = buf(n, "workspace")
        lib.fdec_stub_reserve(ws, B * Hkv * 4)
        if kind == "balanced":
            rc = lib.fdec_decode_balanced(qb, B, Hq, ctypes.byref(kv), lens, nb, 0.0, out, lse, ws, n, None)
        else:
            rc = lib.fdec_decode_multi_balanced(qb, B, ql, Hq, ctypes.byref(kv), lens, nb, 0.0, out, lse, ws, n,
                                                None)
        check(rc, (OK, UNSUPPORTED), what + f" nb={nb}")
        if D == 128 and G in (4, 8) and ql == 1:
            check(rc, (OK,), what + f" nb={nb}")
    elif kind == "multi":
        Su = plan_splits(B, Hq, kv, cap, S)
        n = lib.fdec_workspace_size(B * q_len, Hq, Hkv, D, Su)
        ws = buf(n, "workspace")
        lib.fdec_stub_reserve(ws, B * q_len * Hkv * 4)
        rc = lib.fdec_decode_multi(qb, B, q_len, Hq, ctypes.byref(kv), lens, S, 0.0, out, lse, ws, n, None)
        check(rc, (OK, UNSUPPORTED), what)
        if q_len == 1 or (D == 128 and dtype != 2):
            check(rc, (OK,), what)
    elif kind == "cascade":
        if not paged:
            return
        prefix_len = int(rng.integers(0, 3000))
        pages = buf(((prefix_len + kv.page_size - 1) // kv.page_size) * 4, "prefix_pages")
        sp, ss = int(rng.choice([0, 1, 4, 32])), int(rng.choice([0, 1, 8, 128]))
        psp, pss = I(1), I(1)
        rc = lib.fdec_cascade_plan(B, Hq, Hkv, prefix_len, cap, kv.page_size, 256, ctypes.byref(psp),
                                   ctypes.byref(pss))
        check(rc, (OK,), what + " (plan)")
        n = lib.fdec_cascade_workspace_size(B, Hq, Hkv, D, sp or psp.value, ss or pss.value)
        ws = buf(n, "workspace")
        lib.fdec_stub_reserve(ws, B * Hkv * 4)
        rc = lib.fdec_cascade_decode(qb, B, Hq, ctypes.byref(kv), pages, prefix_len, lens, sp, ss, 0.0, out, lse, ws,
                                     n, None)
        check(rc, (OK, UNSUPPORTED, INVALID), what + f" prefix={prefix_len} sp={sp} ss={ss}")
        if D == 128 and not kv.cache_leftpad and rc != OK:
            msg = lib.fdec_last_error().decode()
            if "too many pages" not in msg and "too many splits" not in msg:
                raise SystemExit(f"{what}: cascade refused: {msg}")
    else:  # argument edge cases: every one returns a status and launches nothing
        for args in [(-1, Hq, 1), (B, 0, 1), (B, Hq, -1), (B, Hq, 300)]:
            rc = lib.fdec_decode(qb, args[0], args[1], ctypes.byref(kv), lens, args[2], 0.0, None, 0, out, lse, None,
                                 0, None)
            check(rc, (INVALID, UNSUPPORTED, WORKSPACE), what + f" args={args}")


def planners(rng):
    out, o2 = I(0), I(0)
    for _ in range(500):
        B = int(rng.integers(0, 300))
        Hkv = int(rng.choice([1, 2, 4, 8, 16]))
        Hq = Hkv * int(rng.choice([1, 2, 4, 8]))
        cap = int(rng.choice([1, 15, 16, 17, 4096, 131072, 1 << 20, (1 << 31) - 1]))
        ps = int(rng.choice([0, 16, 64]))
        lens = np.minimum(rng.integers(0, cap + 1, size=max(B, 1)), cap).astype(np.int32)
        rc = lib.fdec_plan_kv(B, Hq, Hkv, lens.ctypes.data if rng.random() < 0.5 else None, cap, ps,
                              int(rng.choice([0, 1, 2])), int(rng.choice([0, 1, 256, 304])), ctypes.byref(out))
        check(rc, (OK, INVALID), "plan_kv")
        if rc == OK and not (1 <= out.value <= 256):
            raise SystemExit(f"plan_kv gave {out.value}")
        check(lib.fdec_plan_rules(B, Hkv, int(rng.choice([1, 80, 132, 256])), int(rng.choice([1, 64, 128])),
                                  ctypes.byref(out)), (OK, INVALID), "plan_rules")
        lib.fdec_split_chunk(cap, int(rng.choice([1, 2, 7, 256, 0, -3])))
        check(lib.fdec_cascade_plan(B, Hq, Hkv, int(rng.integers(0, 1 << 20)), max(cap, 1), 64, 256,
                                    ctypes.byref(out), ctypes.byref(o2)), (OK, INVALID), "cascade_plan")


def main():
    rng = np.random.default_rng(2024)
    lib.fdec_trace_start(64)
    for i in range(NCASES):
        one_case(rng, i)
    n = I(0)
    check(lib.fdec_trace_stop(None, None, 0, ctypes.byref(n)), (OK,), "trace_stop")
    planners(rng)
    launches = lib.fdec_stub_launches()
    print(f"host sweep ok: {NCASES} cases, {launches} checked launches, {n.value} trace events")
    if launches < NCASES // 2:
        raise SystemExit("too few launches: the sweep is not reaching the launch code")


if __name__ == "__main__":
    main()
