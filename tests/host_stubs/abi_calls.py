"""Drives every C-ABI entry point of a host build of fa_api.cpp whose kernel
launchers are the stand-ins of fa_launch_stubs.cpp, with exact-size host
workspaces, across ragged shapes, every head dim, both masks, both dtypes and
every dQ method.  Run in a process with AddressSanitizer preloaded: an access
past a workspace the library sized, or undefined behaviour in its size and
offset arithmetic, aborts the process.  Prints one line per group of calls
and "ALL OK" at the end; exits non-zero on any unexpected status.

usage: python abi_calls.py <libfa_host.so>
"""
import ctypes as C
import os
import sys

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
BF16, FP32 = 0, 1
HANDOFF, RECOMPUTE, ATOMIC = 0, 1, 2

lib = C.CDLL(sys.argv[1])
vp, sz, i32, f32, u64, u32 = C.c_void_p, C.c_size_t, C.c_int, C.c_float, C.c_ulonglong, C.c_uint
lib.host_workspace.restype = vp
lib.host_workspace.argtypes = [sz]
lib.host_free.argtypes = [vp]
lib.fa_bwd_workspace_size.restype = sz
lib.fa_bwd_workspace_size.argtypes = [i32] * 7
lib.fa_bwd_workspace_bytes.restype = sz
lib.fa_bwd_workspace_bytes.argtypes = [i32] * 5
lib.fa_bwd_dq_method.argtypes = [i32] * 6 + [sz, i32]
lib.fa_fwd.argtypes = [vp] * 5 + [i32] * 5 + [f32, vp, i32, i32]
lib.fa_bwd.argtypes = [vp] * 9 + [i32] * 5 + [f32, vp, sz, vp, i32, i32]
lib.fa_bwd_preprocess.argtypes = [vp] * 3 + [i32] * 4 + [f32, vp, sz, vp, i32, i32]
lib.fa_bwd_dkdv.argtypes = [vp] * 7 + [i32] * 5 + [f32, vp, sz, vp, i32, i32]
lib.fa_bwd_dq.argtypes = [vp] * 6 + [i32] * 5 + [f32, vp, sz, vp, i32, i32]
lib.fa_fwd_dropout.argtypes = [vp] * 5 + [i32] * 5 + [f32, i32, u64, u32, vp, i32]
lib.fa_bwd_dropout.argtypes = [vp] * 9 + [i32] * 5 + [f32, i32, u64, u32, vp, sz, vp, i32]
lib.fa_fwd_fp8.argtypes = [vp] * 5 + [i32] * 5 + [f32] * 4 + [vp, i32]
lib.fa_fwd_splitkv_workspace_bytes.restype = sz
lib.fa_fwd_splitkv_workspace_bytes.argtypes = [i32] * 6
lib.fa_fwd_splitkv.argtypes = [vp] * 5 + [i32] * 6 + [f32, i32, vp, sz, vp, i32, i32]
lib.fa_fwd_splitkv_fp8_workspace_bytes.restype = sz
lib.fa_fwd_splitkv_fp8_workspace_bytes.argtypes = [i32] * 6
lib.fa_fwd_splitkv_fp8.argtypes = [vp] * 5 + [i32] * 6 + [f32] * 4 + [i32, vp, sz, vp, i32]
pll = C.POINTER(C.c_longlong)
lib.fa_fwd_strided.argtypes = [vp] * 5 + [i32] * 5 + [f32, pll, vp, i32]
lib.fa_bwd_strided.argtypes = [vp] * 9 + [i32] * 5 + [f32, pll, vp, sz, vp, i32]
lib.fa_strerror.restype = C.c_char_p
lib.fa_strerror.argtypes = [i32]

# tensors are opaque to the host layer: distinct, aligned, never dereferenced
T = [0x10000 * (i + 1) for i in range(9)]
q, k, v, o, lse, dO, dq, dk, dv = T
fails = []


def expect(got, want, what):
    if got != want:
        fails.append(f"{what}: status {got}, expected {want}")


def with_ws(nbytes, fn):
    ws = lib.host_workspace(nbytes)
    try:
        return fn(ws)
    finally:
        lib.host_free(ws)


SHAPES = [(1, 1, 1), (2, 3, 33), (1, 2, 64), (2, 1, 100), (1, 1, 257), (3, 2, 513)]
n_calls = 0
for d in (64, 96, 128, 256):
    for dtype in (BF16, FP32):
        for causal in (0, 1):
            for B, H, N in SHAPES:
                fwd = lib.fa_fwd(q, k, v, o, lse, B, H, N, d, causal, 0.125, None, dtype, 0)
                if fwd == UNSUPPORTED:
                    continue
                expect(fwd, OK, f"fa_fwd d={d} dt={dtype} c={causal} {B}x{H}x{N}")
                for method in (HANDOFF, RECOMPUTE, ATOMIC):
                    need = lib.fa_bwd_workspace_size(B, H, N, d, causal, dtype, method)
                    if need == 0:
                        continue
                    if method == ATOMIC:
                        os.environ["FA_DQ_MODE"] = "atomic"
                    tag = f"d={d} dt={dtype} c={causal} m={method} {B}x{H}x{N}"
                    got_m = lib.fa_bwd_dq_method(B, H, N, d, causal, dtype, need, 0)
                    expect(got_m, method, "dq_method " + tag)
                    for lay in (0, 1):
                        def run(ws, lay=lay):
                            r = [lib.fa_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, causal, 0.125, ws, need,
                                            None, dtype, lay),
                                 lib.fa_bwd_preprocess(o, dO, lse, B, H, N, d, 0.125, ws, need, None, dtype, lay),
                                 lib.fa_bwd_dkdv(q, k, v, dO, lse, dk, dv, B, H, N, d, causal, 0.125, ws, need,
                                                 None, dtype, lay),
                                 lib.fa_bwd_dq(q, k, v, dO, lse, dq, B, H, N, d, causal, 0.125, ws, need, None,
                                               dtype, lay)]
                            if dtype == BF16 and method != ATOMIC:
                                r.append(lib.fa_bwd_dropout(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, causal,
                                                            0.125, 32, 7, 3, ws, need, None, lay))
                            return r
                        for i, st in enumerate(with_ws(need, run)):
                            expect(st, OK, f"backward call {i} {tag} layout={lay}")
                        n_calls += 5
                    # one byte short: rejected before anything is touched
                    short = with_ws(need - 1, lambda ws: lib.fa_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d,
                                                                   causal, 0.125, ws, need - 1, None, dtype, 0))
                    if method == RECOMPUTE or method == ATOMIC:
                        expect(short, WORKSPACE, "short workspace " + tag)
                    else:
                        expect(short, OK, "hand-off one byte short falls back to recompute " + tag)
                    os.environ.pop("FA_DQ_MODE", None)
print(f"backward: {n_calls} calls", flush=True)

n_split = 0
for d in (64, 96, 128, 256):
    for causal in (0, 1):
        for B, H, Nq, Nk in [(1, 1, 1, 1), (2, 3, 1, 1000), (1, 2, 7, 4097), (2, 1, 64, 64), (1, 1, 5, 300)]:
            for ns in (0, 1, 2, 3, 7, 1024):
                need = lib.fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, ns)
                if need == 0:
                    fails.append(f"split size 0 for d={d} {B}x{H}x{Nq}x{Nk} ns={ns}")
                    continue
                st = with_ws(need, lambda ws: lib.fa_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, causal, 0.125,
                                                                 ns, ws, need, None, BF16, 1))
                expect(st, OK, f"splitkv d={d} c={causal} {B}x{H}x{Nq}x{Nk} ns={ns}")
                st = with_ws(need - 1, lambda ws: lib.fa_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, causal,
                                                                     0.125, ns, ws, need - 1, None, BF16, 1))
                expect(st, WORKSPACE, f"splitkv short d={d} ns={ns}")
                n_split += 2
                need8 = lib.fa_fwd_splitkv_fp8_workspace_bytes(B, H, Nq, Nk, d, ns)
                st = with_ws(need8, lambda ws: lib.fa_fwd_splitkv_fp8(q, k, v, o, lse, B, H, Nq, Nk, d, causal,
                                                                      0.125, 1.0, 1.0, 1.0, ns, ws, need8,
                                                                      None, 0))
                expect(st, OK, f"splitkv fp8 d={d} c={causal} {B}x{H}x{Nq}x{Nk} ns={ns}")
                n_split += 1
        for B, H, N in SHAPES:
            for lay in (0, 1):
                st = lib.fa_fwd_fp8(q, k, v, o, lse, B, H, N, d, causal, 0.125, 1.0, 1.0, 1.0, None, lay)
                expect(st, OK, f"fa_fwd_fp8 d={d} c={causal} {B}x{H}x{N} lay={lay}")
                n_split += 1
print(f"split and FP8 forwards: {n_split} calls", flush=True)

# strided views: accepted layouts run (here: reach the stand-in launchers),
# and every accepted output view is free of overlap, checked by enumerating
# its element offsets on small shapes
def strided(vals):
    return (C.c_longlong * len(vals))(*vals)


def overlaps(B, H, N, d, st):
    seen = set()
    for b in range(B):
        for h in range(H):
            for n in range(N):
                base = b * st[0] + h * st[1] + n * st[2]
                for c in range(d):
                    if base + c in seen:
                        return True
                    seen.add(base + c)
    return False


n_str = n_accepted = 0
for dtype, unit in ((BF16, 8), (FP32, 4)):
    for B, H, N, d in [(2, 3, 33, 64), (1, 2, 5, 96), (3, 1, 2, 128), (1, 1, 1, 64), (1, 2, 9, 256)]:
        packed = [N * 3 * H * d, d, 3 * H * d]        # a slice of [B, N, 3, H, d]
        bhnd = [H * N * d, N * d, d]
        bnhd = [N * H * d, d, H * d]
        padded = [H * N * (d + 2 * unit), N * (d + 2 * unit), d + 2 * unit]
        for combo in ([packed] * 3 + [bhnd], [bnhd] * 4, [padded, packed, bhnd, bnhd],
                      [[0, bhnd[1], bhnd[2]]] * 3 + [bhnd]):   # inputs broadcast over the batch
            vals = [x for t in combo for x in t]
            st = lib.fa_fwd_strided(q, k, v, o, lse, B, H, N, d, 1, 0.125, strided(vals), None, dtype)
            expect(st, OK, f"fwd_strided dt={dtype} {B}x{H}x{N}x{d} {combo}")
            need = lib.fa_bwd_workspace_size(B, H, N, d, 1, dtype, RECOMPUTE)
            bvals = vals[:12] + combo[3] + combo[0] + combo[1] + combo[2]
            st = with_ws(need, lambda ws: lib.fa_bwd_strided(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, 1, 0.125,
                                                             strided(bvals), ws, need, None, dtype))
            want = OK if combo[0][0] != 0 or B == 1 else INVALID   # dq on the broadcast layout overlaps
            expect(st, want, f"bwd_strided dt={dtype} {B}x{H}x{N}x{d} {combo}")
            n_str += 2
        # random output strides: whatever is accepted must not overlap
        import random
        rng = random.Random(1234 + B * 100 + N + d + dtype)
        for _ in range(150):
            so = [rng.choice([0, unit, d, d + unit, H * d, N * d, rng.randrange(0, 4 * N * H * d + 1, unit)])
                  for _ in range(3)]
            vals = bhnd * 3 + so
            st = lib.fa_fwd_strided(q, k, v, o, lse, B, H, N, d, 0, 0.125, strided(vals), None, dtype)
            if st == OK and overlaps(B, H, N, d, so):
                fails.append(f"accepted an overlapping output view {so} for {B}x{H}x{N}x{d}")
            n_accepted += st == OK
            if st not in (OK, INVALID):
                fails.append(f"fwd_strided status {st} for {so}")
            n_str += 1
# stride values at and past the limits: rejected, with no overflow in the checks
for big in (1 << 40, (1 << 40) + 8, 1 << 62, (1 << 63) - 8, -(1 << 63)):
    vals = [big, 64 * 33, 64] + [3 * 33 * 64, 33 * 64, 64] * 3
    lib.fa_fwd_strided(q, k, v, o, lse, 2, 3, 33, 64, 0, 0.125, strided(vals), None, BF16)
    vals = [3 * 33 * 64, 33 * 64, 64] * 3 + [3 * 33 * 64, big, 64]
    lib.fa_fwd_strided(q, k, v, o, lse, 2, 3, 33, 64, 0, 0.125, strided(vals), None, BF16)
    n_str += 2
if n_accepted < 100:
    fails.append(f"only {n_accepted} random output views were accepted: the overlap check proves little")
print(f"strided: {n_str} calls, {n_accepted} random output views accepted", flush=True)

# rejections: arguments the checks must stop before any size arithmetic
expect(lib.fa_fwd(None, k, v, o, lse, 1, 1, 1, 64, 0, 0.125, None, BF16, 0), INVALID, "null q")
expect(lib.fa_fwd(q + 2, k, v, o, lse, 1, 1, 1, 64, 0, 0.125, None, BF16, 0), INVALID, "misaligned q")
expect(lib.fa_fwd(q, k, v, o, lse, 1, 1, 1, 80, 0, 0.125, None, BF16, 0), UNSUPPORTED, "d=80")
for B, H, N in [(0, 1, 1), (1, 0, 1), (1, 1, 0), (-1, 1, 1), (2**31 - 1, 2**31 - 1, 2**31 - 1)]:
    st = lib.fa_fwd(q, k, v, o, lse, B, H, N, 64, 0, 0.125, None, BF16, 0)
    if st == OK and B > 0 and H > 0 and N > 0:
        pass  # a huge shape is a caller's problem only once a kernel runs; the host layer must not overflow
    elif st not in (INVALID, UNSUPPORTED):
        fails.append(f"fa_fwd {B}x{H}x{N}: status {st}")
    lib.fa_bwd_workspace_size(B, H, N, 128, 1, BF16, HANDOFF)
    lib.fa_bwd_workspace_bytes(B, H, N, 128, BF16)
    lib.fa_fwd_splitkv_workspace_bytes(B, H, 1, N, 128, 0)
for s in range(-8, 3):
    lib.fa_strerror(s)
print("rejections done", flush=True)

if fails:
    print("\n".join(fails[:40]))
    print(f"{len(fails)} failures")
    sys.exit(1)
print("ALL OK")
