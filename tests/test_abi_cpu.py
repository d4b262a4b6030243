"""CPU-only checks of the C-ABI library: it loads, exports every entry point
declared in include/dspark.h, sizes its workspace, and rejects bad arguments
on the host before touching a GPU (no compute call is made here)."""
import ctypes as C
import os
import re

import pytest

import draft_verify_sampling_head_amd as D
from draft_verify_sampling_head_amd import _lib as L
from draft_verify_sampling_head_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = C.c_void_p(0x100000)      # never dereferenced: every call below fails validation first


def declared():
    src = open(os.path.join(ROOT, "include", "dspark.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dspark_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    lib = L.load()
    names = declared()
    assert len(names) >= 10
    for nm in names:
        assert hasattr(lib, nm), nm
    assert set(L.EXPORTS) == set(names)


def test_workspace_and_strings():
    assert D.workspace_bytes(0, 1, 1) >= 256
    assert D.workspace_bytes(256, 16, 129280) > 256 * 1010 * 8
    assert D.workspace_bytes(-1, 1, 1) == 0
    lib = L.load()
    for code, name in L.STATUS.items():
        assert lib.dspark_status_string(code).decode() == name
    assert "gfx950" in D._lib.version()


def _draft(R=4, g=7, V=100, r=0, T=1.0, U=FAKE, W1=None, W2t=None, x0=FAKE, x=FAKE, lp=FAKE,
           lse=FAKE, ws=FAKE, ws_bytes=1 << 30, udt=0, wdt=0):
    return L.load().dspark_draft_markov(R, g, V, r, T, 0, 0, U, udt, W1, W2t, wdt, x0, x, lp, lse,
                                        None, ws, ws_bytes, None)


def test_draft_argument_checks():
    assert _draft(R=-1) == INVALID
    assert _draft(g=0) == INVALID
    assert _draft(g=33) == UNSUPPORTED
    assert _draft(V=0) == INVALID
    assert _draft(r=-16) == INVALID
    assert _draft(r=8) == UNSUPPORTED
    assert _draft(r=528) == UNSUPPORTED
    assert _draft(T=-0.5) == INVALID
    assert _draft(T=float("inf")) == INVALID
    assert _draft(T=float("nan")) == INVALID
    assert _draft(U=None) == INVALID
    assert _draft(r=16) == INVALID                      # rank > 0 needs W1 and W2t
    assert _draft(r=16, W1=C.c_void_p(0x100008), W2t=FAKE) == UNSUPPORTED   # misaligned weights
    assert _draft(ws_bytes=100) == WORKSPACE
    assert _draft(udt=7) == INVALID
    assert _draft(R=0, U=None, x0=None, x=None, lp=None, lse=None, ws=None) == OK  # empty batch


def _draft_rnn(R=4, g=7, V=100, r=16, d=32, T=1.0, U=FAKE, W1=FAKE, W2t=FAKE, Wr=FAKE, h=FAKE,
               feat=FAKE, ws=FAKE, ws_bytes=1 << 30, wdt=1, hdt=1):
    return L.load().dspark_draft_rnn(R, g, V, r, d, T, 0, 0, U, 1, W1, W2t, wdt, Wr, h, hdt, FAKE,
                                     FAKE, FAKE, FAKE, None, feat, None, ws, ws_bytes, None)


def test_rnn_argument_checks():
    assert _draft_rnn(r=0) == UNSUPPORTED               # the RNN head needs a rank
    assert _draft_rnn(r=8) == UNSUPPORTED
    assert _draft_rnn(d=0) == INVALID
    assert _draft_rnn(g=33) == UNSUPPORTED
    assert _draft_rnn(T=-1.0) == INVALID
    assert _draft_rnn(Wr=None) == INVALID
    assert _draft_rnn(h=None) == INVALID
    assert _draft_rnn(feat=None) == INVALID
    assert _draft_rnn(hdt=5) == INVALID
    assert _draft_rnn(feat=C.c_void_p(0x100004)) == UNSUPPORTED           # misaligned features
    need = D.rnn_workspace_bytes(4, 7, 100, 16, 32)
    assert need >= D.workspace_bytes(4, 7, 100) + 4 * 7 * 16 * 4 * 4
    assert _draft_rnn(ws_bytes=need - 1) == WORKSPACE
    assert _draft_rnn(R=0, U=None, W1=None, W2t=None, Wr=None, h=None, feat=None, ws=None) == OK
    # the feature verify: a rank is required, and the features replace W1
    lib = L.load()
    args = lambda r, feat: (4, 7, 100, r, 1.0, 0, 0, FAKE, FAKE, FAKE, 1, 1, FAKE, FAKE, FAKE,
                            FAKE, 1, feat, FAKE, 1, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30,
                            None)
    assert lib.dspark_verify_features(*args(0, FAKE)) == UNSUPPORTED
    assert lib.dspark_verify_features(*args(16, None)) == INVALID


def test_confidence_schedule_pack_verify_checks():
    lib = L.load()
    conf = lambda R=2, g=3, d=8, r=0, V=10, h=FAKE, w=FAKE, x=FAKE, c=FAKE: lib.dspark_confidence(
        R, g, d, r, V, h, 0, None, 0, w, 0, None, x, c, None)
    assert conf(d=0) == INVALID
    assert conf(g=40) == UNSUPPORTED
    assert conf(r=16) == INVALID                         # W1 missing
    assert conf(h=None) == INVALID
    assert conf(R=0, h=None) == OK
    sched = lambda R=4, g=4, c=FAKE, sps=FAKE, N_max=100, ell=FAKE: lib.dspark_prefix_schedule(
        R, g, c, sps, N_max, 1, ell, None, None, None, None)
    assert sched(R=-2) == INVALID
    assert sched(N_max=3) == INVALID                     # N_max < R
    assert sched(R=1024, g=17, N_max=10**6) == UNSUPPORTED   # R * gamma > 16384
    assert sched(c=None) == INVALID
    # static verification needs the whole block within N_max
    stat = lambda N_max: lib.dspark_prefix_schedule(4, 4, FAKE, FAKE, N_max, 0, FAKE, None, None,
                                                     None, None)
    assert stat(19) == INVALID and stat(4) == INVALID
    asch = lambda R=4, g=4, N_max=100, kin=FAKE, kp=FAKE, ell=FAKE: lib.dspark_async_schedule(
        R, g, FAKE, FAKE, N_max, kin, kp, ell, None, None, None, None, None)
    assert asch(R=-1) == INVALID
    assert asch(N_max=3) == INVALID
    assert asch(kin=None) == INVALID and asch(kp=None) == INVALID
    assert asch(g=33) == UNSUPPORTED
    assert asch(R=1024, g=17, N_max=10**6) == UNSUPPORTED
    assert asch(R=0, kin=None) == OK
    sp = lambda R=4, g=4, mode=1, N_max=100, x=FAKE, kin=FAKE, kp=FAKE, cu=FAKE, flat=FAKE: \
        lib.dspark_schedule_pack(R, g, mode, FAKE, FAKE, N_max, kin, kp, x, FAKE, None, None, None,
                                 None, cu, flat, None, None, None)
    assert sp(mode=3) == INVALID and sp(mode=-1) == INVALID
    assert sp(x=None) == INVALID and sp(cu=None) == INVALID and sp(flat=None) == INVALID
    assert sp(N_max=3) == INVALID
    assert sp(mode=0, N_max=19) == INVALID                # static needs the whole block
    assert sp(mode=2, kin=None) == INVALID and sp(mode=2, kp=None) == INVALID
    assert sp(g=33) == UNSUPPORTED
    assert sp(R=1024, g=17, N_max=10**6) == UNSUPPORTED
    assert sp(R=0, x=None) == OK
    pack = lambda R=4, width=3, rows=FAKE, ln=FAKE, cu=FAKE, flat=FAKE: lib.dspark_pack(
        R, width, rows, ln, 0, cu, flat, None, None, None, None, 0, None)
    assert pack(width=0) == INVALID
    assert pack(rows=None) == INVALID
    assert pack(R=1 << 20, width=1 << 12) == UNSUPPORTED
    ver = lambda layout=1, tdt=1, udt=1, T=1.0, ws_bytes=1 << 30, ell=FAKE: lib.dspark_verify(
        4, 3, 100, 0, T, 0, 0, ell, FAKE, FAKE, tdt, layout, FAKE, FAKE, FAKE, FAKE, udt, None,
        None, 1, FAKE, FAKE, FAKE, FAKE, None, FAKE, ws_bytes, None)
    assert ver(layout=2) == INVALID
    assert ver(tdt=0, udt=1) == UNSUPPORTED
    assert ver(T=-1.0) == INVALID
    assert ver(ws_bytes=10) == WORKSPACE
    assert ver(ell=None) == INVALID
    grid = (C.c_float * 3)(0.5, 1.0, 2.0)
    sts = lambda n=10, g=3, G=3, nb=15, gr=grid, wsb=1 << 20: lib.dspark_sts_fit(
        n, g, FAKE, FAKE, C.cast(gr, C.c_void_p), G, nb, FAKE, None, FAKE, wsb, None)
    assert sts(n=0) == INVALID and sts(G=0) == INVALID and sts(nb=0) == INVALID
    assert sts(G=257) == UNSUPPORTED and sts(nb=65) == UNSUPPORTED
    assert sts(gr=(C.c_float * 3)(0.5, -1.0, 2.0)) == INVALID
    assert sts(wsb=64) == WORKSPACE
    assert lib.dspark_sts_workspace_bytes(1000) >= 8000
    acc = lambda T=1.0, R=4, tdt=1: lib.dspark_acceptance_rate(
        R, 3, 100, 0, T, FAKE, tdt, FAKE, FAKE, FAKE, 1, None, None, 1, FAKE, FAKE, 1 << 30, None)
    assert acc(T=-1.0) == INVALID and acc(tdt=0) == UNSUPPORTED and acc(R=0) == OK
    capv = lambda cap=FAKE, R=4: lib.dspark_verify_cap_accept(
        R, 3, 100, 0, 1.0, 0, 0, FAKE, cap, FAKE, FAKE, 1, 1, FAKE, FAKE, FAKE, FAKE, 1, None,
        None, 1, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 30, None)
    assert capv(cap=None) == INVALID
    assert capv(cap=None, R=0) == OK
    tiers = (C.c_int32 * 3)(4, 8, 8)
    ptier = lambda n=3, slots=16, t=tiers, R=4: lib.dspark_pack_tiered(
        R, 3, FAKE, FAKE, 0, C.cast(t, C.c_void_p), n, 0, slots, FAKE, FAKE, None, None,
        None, None, None, 0, None)
    assert ptier() == INVALID                            # tiers not strictly ascending
    assert ptier(n=2, slots=11) == INVALID               # slots < R * width
    assert ptier(n=2, slots=7) == INVALID
    assert ptier(n=33) == UNSUPPORTED
    big = (C.c_int32 * 2)(4, 20)
    assert ptier(n=2, t=big) == INVALID                  # a tier beyond the slots
    assert ptier(n=-1) == INVALID


def test_synthetic_configs_shapes():
    for idx in range(4):
        cfg = synth.config(idx)
        assert cfg.R * cfg.gamma <= 16384 and cfg.rank % 16 == 0
    c4 = synth.config(4, R=512, gamma=16, rank=0)
    assert c4.V == synth.VOCAB_DEEPSEEK and c4.rank == 0
    small = synth.scaled(synth.config(3), R=10, gamma=4, V=300, d=16)
    inp = synth.make_inputs(small, device="cpu")
    assert inp["U"].shape == (10, 4, 300) and inp["target"].shape == (10, 5, 300)
    assert int(inp["hard"].sum()) == 3
    sps = synth.sps_table(synth.config(3), 3000)
    assert sps[0] == sps[31] and sps[2049] == 0 and (sps[32:2049].diff() <= 0).all()


@pytest.mark.parametrize("fn", ["draft_markov", "confidence", "prefix_schedule", "async_schedule",
                                "pack", "pack_tiered", "verify", "verify_cap_accept",
                                "acceptance_rate", "sts_fit", "confidence_logits", "draft_rnn",
                                "verify_features", "rnn_workspace_bytes",
                                "acceptance_rate_features", "verify_cap_accept_features",
                                "schedule_pack", "round_markov"])
def test_binding_names_match_abi(fn):
    assert callable(getattr(D, fn))
    assert f"dspark_{fn}" in declared()


def test_switches_set_get_and_reject():
    """The test switches: known keys round-trip, unknown keys and values are
    rejected, and every switch is restored."""
    keys = [L.SWITCH_FORCE_PER_STEP, L.SWITCH_RNN_CELL_VALU, L.SWITCH_BARRIER_SPINS,
            L.SWITCH_DRAFT_KERNEL, L.SWITCH_PERSIST_LAUNCH]
    saved = [L.get_switch(k) for k in keys]
    try:
        for k in keys:
            assert L.get_switch(k) >= 0
        L.set_switch(L.SWITCH_FORCE_PER_STEP, 1)
        assert L.get_switch(L.SWITCH_FORCE_PER_STEP) == 1
        L.set_switch(L.SWITCH_BARRIER_SPINS, 12345)
        assert L.get_switch(L.SWITCH_BARRIER_SPINS) == 12345
        lib = L.load()
        assert lib.dspark_set_switch(L.SWITCH_FORCE_PER_STEP, 2) == INVALID
        assert lib.dspark_set_switch(L.SWITCH_DRAFT_KERNEL, -1) == INVALID
        assert lib.dspark_set_switch(L.SWITCH_BARRIER_SPINS, -5) == INVALID
        assert lib.dspark_set_switch(L.SWITCH_PERSIST_LAUNCH, 2) == INVALID
        L.set_switch(L.SWITCH_PERSIST_LAUNCH, 1)
        assert L.get_switch(L.SWITCH_PERSIST_LAUNCH) == 1
        assert lib.dspark_set_switch(99, 0) == INVALID
        assert lib.dspark_get_switch(99) == -1
    finally:
        for k, v in zip(keys, saved):
            L.set_switch(k, v)
    assert [L.get_switch(k) for k in keys] == saved


def test_w2_transpose_argument_checks():
    lib = L.load()
    assert lib.dspark_w2_transpose(-1, 10, FAKE, FAKE, 1, None) == INVALID
    assert lib.dspark_w2_transpose(16, 0, FAKE, FAKE, 1, None) == INVALID
    assert lib.dspark_w2_transpose(16, 10, FAKE, FAKE, 7, None) == INVALID     # unknown dtype
    assert lib.dspark_w2_transpose(16, 10, None, FAKE, 1, None) == INVALID
    assert lib.dspark_w2_transpose(16, 10, FAKE, FAKE, 1, None) == INVALID     # same buffer
    assert lib.dspark_w2_transpose(0, 10, None, None, 1, None) == OK           # r == 0: nothing


def test_every_enqueueing_entry_point_has_a_marker_range():
    """Each C-ABI call that takes a stream (and the blocking status read) opens
    a roctx range named after itself, and the library links the roctx
    runtime."""
    csrc = os.path.join(ROOT, "draft_verify_sampling_head_amd", "csrc")
    found = {}
    for fn in sorted(os.listdir(csrc)):
        if not fn.endswith(".hip"):
            continue
        src = open(os.path.join(csrc, fn)).read()
        for m in re.finditer(r'^(?:extern "C" )?dspark_status (dspark_\w+)\(', src, re.M):
            body = src.index(") {", m.end())
            sig = src[m.start():body]
            first = src[body + 3:].lstrip().split("\n", 1)[0]
            if "hipStream_t" in sig or m.group(1) == "dspark_get_status":
                found[m.group(1)] = first.strip() == "DSPARK_ABI_RANGE();"
    assert "dspark_verify" in found and "dspark_draft_markov_noalloc" in found
    assert all(found.values()), [k for k, v in found.items() if not v]
    assert set(found) <= set(declared())
    with open(L.LIB_PATH, "rb") as f:
        assert b"librocprofiler-sdk-roctx.so" in f.read()


def _round(**kw):
    A = L.RoundMarkovArgs()
    A.R, A.gamma, A.V, A.r, A.d, A.T = 4, 7, 100, 0, 32, 1.0
    A.sched_mode, A.N_max, A.target_layout = 1, 4 * 8, 1
    for n, _ in L.RoundMarkovArgs._fields_:
        if n not in ("R", "gamma", "V", "r", "d", "T", "seed", "round", "sched_mode", "N_max",
                     "target_layout") and not n.endswith("_dt"):
            setattr(A, n, FAKE.value)
    for n, v in kw.items():
        setattr(A, n, v)
    return L.load().dspark_round_markov(C.byref(A), FAKE, 1 << 30, None)


def test_round_markov_checks_every_call_before_enqueueing():
    """The one-call round rejects what any of its five calls would reject.
    Errors found by the later calls' checks come back as those calls' codes:
    had the draft been enqueued first, the launch (no GPU here) would have
    failed with DSPARK_E_HIP instead."""
    lib = L.load()
    assert lib.dspark_round_markov(None, FAKE, 1 << 30, None) == INVALID
    assert _round(sched_mode=3) == INVALID
    assert _round(gamma=33) == UNSUPPORTED              # draft
    assert _round(h=None) == INVALID                    # confidence
    assert _round(N_max=3) == INVALID                   # schedule: N_max < R
    assert _round(sched_mode=0, N_max=31) == INVALID    # static block needs R (gamma + 1)
    assert _round(sched_mode=2, K_in=None) == INVALID   # asynchronous scheduler needs K_in
    assert _round(t_dt=1) == UNSUPPORTED                # verify: target and U dtypes differ
    assert _round(target_layout=2) == INVALID           # verify
    assert _round(cu_out=None) == INVALID               # output pack
    assert lib.dspark_round_markov(C.byref(L.RoundMarkovArgs()), FAKE, 1 << 30, None) == INVALID
    assert _round(R=0) == OK                            # empty batch: nothing to do


def test_round_markov_args_layout_matches_header(tmp_path):
    """The binding's ctypes mirror of dspark_round_markov_args has the C
    struct's size and every field at the C offset (a small C program compiled
    against include/dspark.h prints them)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    fields = [n for n, _ in L.RoundMarkovArgs._fields_]
    hip_stub = tmp_path / "hip" / "hip_runtime_api.h"
    hip_stub.parent.mkdir()
    hip_stub.write_text("typedef struct ihipStream_t* hipStream_t;\n"
                        "typedef struct ihipEvent_t* hipEvent_t;\n")
    src = tmp_path / "layout.c"
    body = "\n".join(f'  printf("{n} %zu\\n", offsetof(dspark_round_markov_args, {n}));' for n in fields)
    src.write_text("#include <stddef.h>\n#include <stdio.h>\n#include \"dspark.h\"\n"
                   "int main(void) {\n"
                   '  printf("sizeof %zu\\n", sizeof(dspark_round_markov_args));\n'
                   f"{body}\n  return 0;\n}}\n")
    exe = tmp_path / "layout"
    r = subprocess.run([cc, "-std=c11", f"-I{tmp_path}", f"-I{os.path.join(ROOT, 'include')}",
                        str(src), "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                       check=True).stdout.splitlines())
    assert int(out["sizeof"]) == C.sizeof(L.RoundMarkovArgs)
    for n in fields:
        assert int(out[n]) == getattr(L.RoundMarkovArgs, n).offset, n
