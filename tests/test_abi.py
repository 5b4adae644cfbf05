"""The C ABI on the CPU: the library loads, exports every function include/gdn.h
declares, and rejects bad arguments on the host before any HIP call.

No call here reaches a kernel launch: every case carries an invalid argument,
and the calls run in a child process that sees no GPU (HIP_VISIBLE_DEVICES and
ROCR_VISIBLE_DEVICES hide every device), so even an unexpected pass of the
validation could only end in a launch error, never in device work.
"""
import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")
LIB = os.path.join(ROOT, "linear_attention_recurrence_step_amd", "libgdn.so")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_three_entry_points():
    fns = _declared_functions()
    for name in ("gdn_record", "gdn_replay", "gqa_expand", "gdn_prefill", "gdn_prefill_workspace_size",
                 "rms_norm_bf16", "gdn_record_debug", "gdn_replay_debug", "gdn_prefill_noalloc",
                 "gdn_strerror", "gdn_last_error", "gdn_abi_version"):
        assert name in fns, fns


def test_library_exports_every_declared_function():
    assert os.path.exists(LIB), "libgdn.so is not built"
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = [f for f in _declared_functions() if f not in exported]
    assert not missing, missing


CHILD = r"""
import ctypes, json, sys
lib = ctypes.CDLL(sys.argv[1])
vp, u32, i32 = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_int
lib.gdn_record.argtypes = [vp] * 12 + [u32] * 6 + [i32, i32, vp]
lib.gdn_replay.argtypes = [vp] * 6 + [u32] * 6 + [i32, vp]
lib.gqa_expand.argtypes = [vp, vp] + [u32] * 4 + [i32, i32, vp]
lib.rms_norm_bf16.argtypes = [vp, vp, vp, u32, u32, ctypes.c_float, vp]
lib.gdn_prefill.argtypes = [vp] * 13 + [ctypes.c_uint64] + [u32] * 6 + [i32, i32, vp]
lib.gdn_prefill_noalloc.argtypes = [vp] * 12 + [u32] * 6 + [i32, i32, vp]
lib.gdn_prefill_workspace_size.argtypes = [u32] * 3
lib.gdn_prefill_workspace_size.restype = ctypes.c_uint64
class Choice(ctypes.Structure):
    _fields_ = [("rows_per_thread", ctypes.c_uint32), ("threads", ctypes.c_uint32),
                ("replay_fold", ctypes.c_int32), ("matrix_waves", ctypes.c_uint32)]
lib.gdn_record_debug.argtypes = [ctypes.POINTER(Choice)] + lib.gdn_record.argtypes
lib.gdn_replay_debug.argtypes = [ctypes.POINTER(Choice)] + lib.gdn_replay.argtypes
lib.gdn_strerror.restype = ctypes.c_char_p
lib.gdn_last_error.restype = ctypes.c_char_p
cases = json.loads(sys.argv[2])
out = []
for c in cases:
    fn = getattr(lib, c["fn"])
    args = [None if a is None else a for a in c["args"]]
    if c["fn"].endswith("_debug"):
        ch = c["args"][0]
        args[0] = None if ch is None else ctypes.byref(Choice(*ch))
    rc = fn(*args)
    out.append({"id": c["id"], "rc": rc, "msg": lib.gdn_last_error().decode()})
out.append({"id": "strerror", "rc": 0,
            "msg": json.dumps({str(s): lib.gdn_strerror(s).decode() for s in range(-11, 1)})})
out.append({"id": "ws_size", "rc": 0,
            "msg": json.dumps([lib.gdn_prefill_workspace_size(*x) for x in ([1, 4096, 32], [2, 65, 3], [1, 1, 1],
                                                                             [0xFFFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF])])})
print(json.dumps(out))
"""

BASE = 1 << 40
SPAN = 1 << 36


def P(i, off=0):
    """A distinct, 256-byte aligned fake device address (never dereferenced)."""
    return BASE + i * SPAN + off


# gdn_record(q, k, v, g, beta, state_in, mask, y, state_out, delta_log, k_log, g_log,
#            B, T, Hk, Hv, Dk, Dv, io, map, stream)
def rec(**kw):
    a = dict(q=P(0), k=P(1), v=P(2), g=P(3), beta=P(4), s_in=P(5), mask=P(6), y=P(7), s_out=P(8),
             dl=P(9), kl=P(10), gl=P(11), B=2, T=3, Hk=2, Hv=4, Dk=128, Dv=128, io=2, map=0)
    a.update(kw)
    return [a["q"], a["k"], a["v"], a["g"], a["beta"], a["s_in"], a["mask"], a["y"], a["s_out"],
            a["dl"], a["kl"], a["gl"], a["B"], a["T"], a["Hk"], a["Hv"], a["Dk"], a["Dv"], a["io"],
            a["map"], None]


# gdn_replay(delta_log, k_log, g_log, state_in, mask, state_out, B, T_log, Hv, Dk, Dv, accepted, io, stream)
def rep(**kw):
    a = dict(dl=P(0), kl=P(1), gl=P(2), s_in=P(3), mask=P(4), s_out=P(5), B=2, T=3, Hv=4, Dk=128,
             Dv=128, acc=2, io=1)
    a.update(kw)
    return [a["dl"], a["kl"], a["gl"], a["s_in"], a["mask"], a["s_out"], a["B"], a["T"], a["Hv"],
            a["Dk"], a["Dv"], a["acc"], a["io"], None]


# gqa_expand(src, dst, seq, hg, h, k, dtype, map, stream)
def exp(**kw):
    a = dict(src=P(0), dst=P(1), seq=4, hg=2, h=4, k=128, dt=0, map=1)
    a.update(kw)
    return [a["src"], a["dst"], a["seq"], a["hg"], a["h"], a["k"], a["dt"], a["map"], None]


# rms_norm_bf16(x, weight, out, n_tokens, dim, eps, stream)
def rms(**kw):
    a = dict(x=P(0), w=P(1), out=P(2), n=8, dim=2048, eps=1e-6)
    a.update(kw)
    return [a["x"], a["w"], a["out"], a["n"], a["dim"], a["eps"], None]


# gdn_prefill(q, k, v, g, beta, state_in, mask, y, state_out, delta_log, k_log, g_log, workspace,
#             workspace_bytes, B, T, Hk, Hv, Dk, Dv, io, map, stream)
WS_NEED = 2 * 4 * 1 * 33280          # B=2, Hv=4, one chunk of 64 steps


def pre(**kw):
    a = dict(q=P(0), k=P(1), v=P(2), g=P(3), beta=P(4), s_in=P(5), mask=P(6), y=P(7), s_out=P(8),
             dl=P(9), kl=P(11), gl=P(12), ws=P(10), wsb=WS_NEED, B=2, T=3, Hk=2, Hv=4, Dk=128,
             Dv=128, io=2, map=1)
    a.update(kw)
    return [a["q"], a["k"], a["v"], a["g"], a["beta"], a["s_in"], a["mask"], a["y"], a["s_out"],
            a["dl"], a["kl"], a["gl"], a["ws"], a["wsb"], a["B"], a["T"], a["Hk"], a["Hv"], a["Dk"],
            a["Dv"], a["io"], a["map"], None]


# gdn_record_debug / gdn_replay_debug: the launch choice first, as
# [rows_per_thread, threads, replay_fold, matrix_waves] (None: NULL)
def recd(choice, **kw):
    return [choice] + rec(**kw)


def repd(choice, **kw):
    return [choice] + rep(**kw)


# gdn_prefill_noalloc: gdn_prefill's arguments less workspace and workspace_bytes
def prena(**kw):
    a = pre(**kw)
    return a[:12] + a[14:]


NULL, ZERO, RATIO, SHAPE, OVER, ALIAS, ENUM, LAUNCH, ALIGN = -1, -2, -3, -4, -5, -6, -7, -8, -9
WORKSPACE = -10

CASES = [
    ("rec_bad_dtype", "gdn_record", rec(io=3), ENUM),
    ("rec_bad_map", "gdn_record", rec(map=2), ENUM),
    ("rec_null_q", "gdn_record", rec(q=None), NULL),
    ("rec_null_state_out", "gdn_record", rec(s_out=None), NULL),
    ("rec_zero_B", "gdn_record", rec(B=0), ZERO),
    ("rec_zero_T", "gdn_record", rec(T=0), ZERO),
    ("rec_ratio", "gdn_record", rec(Hk=3, Hv=4), RATIO),
    ("rec_dk48", "gdn_record", rec(Dk=48), SHAPE),
    ("rec_dk512", "gdn_record", rec(Dk=512), SHAPE),
    ("rec_dv40", "gdn_record", rec(Dv=40), SHAPE),
    ("rec_dv2048", "gdn_record", rec(Dv=2048), SHAPE),
    ("rec_bytes_overflow", "gdn_record", rec(B=1 << 31, T=1 << 31), OVER),
    ("rec_grid_overflow", "gdn_record", rec(B=1 << 20, T=1, Hk=1 << 12, Hv=1 << 12, Dk=32, Dv=16), OVER),
    # 2^30 state rows: 2^25 workgroups of 256 threads, 2^33 threads in one launch
    ("rec_work_items_overflow", "gdn_record", rec(B=1 << 20, T=1, Hk=1, Hv=1, Dk=32, Dv=1024), OVER),
    ("rep_work_items_overflow", "gdn_replay", rep(B=1 << 20, T=1, Hv=1, Dk=32, Dv=1024, acc=1), OVER),
    ("rec_misaligned_q", "gdn_record", rec(q=P(0, 2)), ALIGN),
    ("rec_misaligned_state", "gdn_record", rec(s_in=P(5, 8)), ALIGN),
    ("rec_misaligned_mask", "gdn_record", rec(mask=P(6, 2)), ALIGN),
    ("rec_misaligned_g", "gdn_record", rec(g=P(3, 1)), ALIGN),
    ("rec_y_overlaps_v", "gdn_record", rec(y=P(2, 256)), ALIAS),
    ("rec_state_partial_alias", "gdn_record", rec(s_out=P(5, 4096)), ALIAS),
    ("rec_delta_overlaps_y", "gdn_record", rec(dl=P(7, 64)), ALIAS),
    ("rec_state_out_over_q", "gdn_record", rec(s_out=P(0)), ALIAS),
    ("rec_y_over_mask", "gdn_record", rec(y=P(6)), ALIAS),
    ("rec_k_log_over_k", "gdn_record", rec(kl=P(1, 512)), ALIAS),
    ("rec_g_log_over_delta", "gdn_record", rec(gl=P(9, 2)), ALIAS),
    ("rec_k_log_over_y", "gdn_record", rec(kl=P(7)), ALIAS),
    ("rec_misaligned_k_log", "gdn_record", rec(kl=P(10, 8)), ALIGN),
    ("rec_misaligned_g_log", "gdn_record", rec(gl=P(11, 1)), ALIGN),
    ("rec_k_log_bytes_overflow", "gdn_record", rec(B=1 << 20, T=1 << 20, Hk=1, Hv=1 << 12), OVER),
    ("rep_bad_dtype", "gdn_replay", rep(io=-1), ENUM),
    ("rep_null_k_log", "gdn_replay", rep(kl=None), NULL),
    ("rep_zero_T", "gdn_replay", rep(T=0), ZERO),
    ("rep_zero_Dv", "gdn_replay", rep(Dv=0), ZERO),
    ("rep_dk96", "gdn_replay", rep(Dk=96), SHAPE),
    ("rep_misaligned_delta", "gdn_replay", rep(dl=P(0, 4)), ALIGN),
    ("rep_state_out_over_tape", "gdn_replay", rep(s_out=P(0, 1024)), ALIAS),
    ("rep_state_partial_alias", "gdn_replay", rep(s_out=P(3, 16)), ALIAS),
    ("rep_bytes_overflow", "gdn_replay", rep(B=1 << 31, T=1 << 31), OVER),
    ("rms_null_x", "rms_norm_bf16", rms(x=None), NULL),
    ("rms_null_weight", "rms_norm_bf16", rms(w=None), NULL),
    ("rms_null_out", "rms_norm_bf16", rms(out=None), NULL),
    ("rms_zero_dim", "rms_norm_bf16", rms(dim=0), ZERO),
    ("rms_zero_tokens", "rms_norm_bf16", rms(n=0), ZERO),
    ("rms_misaligned_x", "rms_norm_bf16", rms(x=P(0, 2)), ALIGN),
    ("rms_misaligned_out", "rms_norm_bf16", rms(out=P(2, 6)), ALIGN),
    ("rms_misaligned_weight", "rms_norm_bf16", rms(w=P(1, 1)), ALIGN),
    ("rms_out_overlaps_x", "rms_norm_bf16", rms(out=P(0, 16)), ALIAS),
    ("rms_out_overlaps_weight", "rms_norm_bf16", rms(out=P(1, 64)), ALIAS),
    ("rms_bytes_overflow", "rms_norm_bf16", rms(n=1 << 31, dim=1 << 20), OVER),
    ("pre_bad_dtype", "gdn_prefill", pre(io=5), ENUM),
    ("pre_bad_map", "gdn_prefill", pre(map=3), ENUM),
    ("pre_null_v", "gdn_prefill", pre(v=None), NULL),
    ("pre_zero_T", "gdn_prefill", pre(T=0), ZERO),
    ("pre_ratio", "gdn_prefill", pre(Hk=3), RATIO),
    ("pre_dk256", "gdn_prefill", pre(Dk=256), SHAPE),
    ("pre_f32", "gdn_prefill", pre(io=0), SHAPE),
    ("pre_dk64", "gdn_prefill", pre(Dk=64), SHAPE),
    ("pre_dv40", "gdn_prefill", pre(Dv=40), SHAPE),
    ("pre_dv2048", "gdn_prefill", pre(Dv=2048), SHAPE),
    ("pre_null_workspace", "gdn_prefill", pre(ws=None), WORKSPACE),
    ("pre_short_workspace", "gdn_prefill", pre(wsb=WS_NEED - 1), WORKSPACE),
    ("pre_short_workspace_T65", "gdn_prefill", pre(T=65), WORKSPACE),
    ("pre_misaligned_workspace", "gdn_prefill", pre(ws=P(10, 16)), ALIGN),
    ("pre_misaligned_q", "gdn_prefill", pre(q=P(0, 8)), ALIGN),
    ("pre_workspace_over_k", "gdn_prefill", pre(ws=P(1)), ALIAS),
    ("pre_workspace_over_y", "gdn_prefill", pre(ws=P(7, 256)), ALIAS),
    ("pre_y_over_v", "gdn_prefill", pre(y=P(2, 512)), ALIAS),
    ("pre_state_partial_alias", "gdn_prefill", pre(s_out=P(5, 4096)), ALIAS),
    ("pre_grid_overflow", "gdn_prefill", pre(B=1 << 16, T=1 << 15, Hk=1, Hv=1 << 8, Dv=16), OVER),
    ("pre_k_log_over_k", "gdn_prefill", pre(kl=P(1, 512)), ALIAS),
    ("pre_g_log_over_workspace", "gdn_prefill", pre(gl=P(10, 64)), ALIAS),
    ("pre_k_log_over_g_log", "gdn_prefill", pre(gl=P(11, 256)), ALIAS),
    ("pre_misaligned_k_log", "gdn_prefill", pre(kl=P(11, 8)), ALIGN),
    ("pre_misaligned_g_log", "gdn_prefill", pre(gl=P(12, 1)), ALIGN),
    ("pre_k_log_bytes_overflow", "gdn_prefill", pre(B=1 << 20, T=1 << 20, Hk=1, Hv=1 << 12), OVER),
    ("recd_unknown_tiling", "gdn_record_debug", recd([3, 256, 0, 0]), ENUM),
    ("recd_half_tiling", "gdn_record_debug", recd([2, 0, 0, 0]), ENUM),
    ("recd_huge_tiling", "gdn_record_debug", recd([1 << 31, 256, 0, 0]), ENUM),
    ("recd_replay_fold_on_record", "gdn_record_debug", recd([0, 0, 1, 0]), ENUM),
    ("recd_waves_on_record", "gdn_record_debug", recd([0, 0, 0, 4]), ENUM),
    # 128 rows per workgroup: fine for one step, too many for the staged kernel
    ("recd_staged_too_many_rows", "gdn_record_debug", recd([8, 256, 0, 0], T=3), SHAPE),
    ("recd_rows_not_dividing_dv", "gdn_record_debug", recd([2, 256, 0, 0], T=1, Dv=48), SHAPE),
    ("recd_too_many_state_values", "gdn_record_debug", recd([8, 256, 0, 0], T=1, Dk=192), SHAPE),
    ("recd_null_choice_still_validates", "gdn_record_debug", recd(None, q=None), NULL),
    ("repd_bad_fold", "gdn_replay_debug", repd([0, 0, 3, 0]), ENUM),
    ("repd_bad_waves", "gdn_replay_debug", repd([0, 0, 2, 3]), ENUM),
    ("repd_matrix_on_f32", "gdn_replay_debug", repd([0, 0, 2, 0], io=0), SHAPE),
    ("repd_matrix_dv48", "gdn_replay_debug", repd([0, 0, 2, 0], Dv=48), SHAPE),
    ("repd_tiling_not_fitting", "gdn_replay_debug", repd([8, 256, 1, 0], Dv=64), SHAPE),
    ("repd_unknown_tiling", "gdn_replay_debug", repd([4, 64, 1, 0]), ENUM),
    ("repd_null_state_out", "gdn_replay_debug", repd([0, 0, 1, 0], s_out=None), NULL),
    ("prena_bad_dtype", "gdn_prefill_noalloc", prena(io=5), ENUM),
    ("prena_null_q", "gdn_prefill_noalloc", prena(q=None), NULL),
    ("prena_f32", "gdn_prefill_noalloc", prena(io=0), SHAPE),
    ("prena_y_over_v", "gdn_prefill_noalloc", prena(y=P(2, 512)), ALIAS),
    ("prena_k_log_over_q", "gdn_prefill_noalloc", prena(kl=P(0, 16)), ALIAS),
    ("prena_misaligned_g_log", "gdn_prefill_noalloc", prena(gl=P(12, 1)), ALIGN),
    # one chunk block past the 2048 the scratch area holds
    ("prena_past_scratch", "gdn_prefill_noalloc", prena(B=1, T=64 * 65, Hk=1, Hv=32), WORKSPACE),
    ("prena_past_scratch_batch", "gdn_prefill_noalloc", prena(B=2049, T=1, Hk=1, Hv=1), WORKSPACE),
    ("exp_bad_dtype", "gqa_expand", exp(dt=7), ENUM),
    ("exp_bad_map", "gqa_expand", exp(map=-1), ENUM),
    ("exp_null_dst", "gqa_expand", exp(dst=None), NULL),
    ("exp_zero_k", "gqa_expand", exp(k=0), ZERO),
    ("exp_zero_seq", "gqa_expand", exp(seq=0), ZERO),
    ("exp_ratio", "gqa_expand", exp(hg=3, h=4), RATIO),
    ("exp_overlap", "gqa_expand", exp(dst=P(0, 512)), ALIAS),
    ("exp_misaligned", "gqa_expand", exp(dst=P(1, 2), dt=0), ALIGN),
    ("exp_overflow", "gqa_expand", exp(seq=0xFFFFFFFF, h=0xFFFFFFFF, hg=1, k=0xFFFFFFFF), OVER),
]


@pytest.fixture(scope="module")
def results():
    cases = [{"id": i, "fn": f, "args": a} for i, f, a, _ in CASES]
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1",
               CUDA_VISIBLE_DEVICES="-1")
    r = subprocess.run([sys.executable, "-c", CHILD, LIB, json.dumps(cases)], capture_output=True,
                       text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stderr
    return {d["id"]: d for d in json.loads(r.stdout.strip().splitlines()[-1])}


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_invalid_arguments_are_rejected_before_any_hip_call(results, case):
    cid, fn, _, want = case
    got = results[cid]
    assert got["rc"] == want, (cid, got)
    assert got["msg"].startswith(fn + ":"), got["msg"]


def test_strerror_covers_every_status(results):
    table = json.loads(results["strerror"]["msg"])
    for s in range(-10, 1):
        assert table[str(s)] and table[str(s)] != "unknown status", s
    assert table["-11"] == "unknown status"


def test_prefill_workspace_size(results):
    """33280 bytes per (batch row, value head, chunk of 64 steps)."""
    assert json.loads(results["ws_size"]["msg"]) == [32 * 64 * 33280, 2 * 3 * 2 * 33280, 33280,
                                                     2 ** 64 - 1]   # saturates instead of wrapping


def test_python_binding_names_match_the_abi():
    import linear_attention_recurrence_step_amd as gdn
    from linear_attention_recurrence_step_amd import _native
    for name in ("gdn_record", "gdn_replay", "gqa_expand", "gdn_prefill", "gdn_prefill_workspace_size",
                 "rms_norm_bf16", "gdn_record_debug", "gdn_replay_debug", "gdn_prefill_noalloc"):
        assert callable(getattr(gdn, name))
        assert hasattr(_native.lib, name)
    assert _native.lib.gdn_abi_version() == _native.ABI_VERSION
    assert set(_native.EXPORTS) <= set(_declared_functions())


def test_python_binding_rejects_host_tensors_before_the_library():
    """Well-formed host tensors must never reach the library (a host pointer in a
    kernel would fault the device)."""
    import torch
    import linear_attention_recurrence_step_amd as gdn
    q = torch.zeros(1, 1, 1, 32)
    v = torch.zeros(1, 1, 1, 32)
    g = torch.zeros(1, 1, 1)
    s = torch.zeros(1, 1, 32, 32)
    with pytest.raises(ValueError, match="HIP device"):
        gdn.gdn_record(q, q, v, g, g, s)
    with pytest.raises(ValueError, match="HIP device"):
        gdn.gdn_replay(v, q, g, s, None, 1)
    with pytest.raises(ValueError, match="HIP device"):
        gdn.gdn_prefill(q, q, v, g, g, s)
    with pytest.raises(ValueError, match="HIP device"):
        gdn.gqa_expand(torch.zeros(2, 1, 32), 2)
    with pytest.raises(ValueError, match="HIP device"):
        gdn.rms_norm_bf16(torch.zeros(2, 32), torch.zeros(32, dtype=torch.bfloat16), 1e-6)


def test_library_reads_no_environment():
    """What a call runs depends on its arguments only: the library's sources
    read no environment variable."""
    import glob
    for path in glob.glob(os.path.join(ROOT, "linear_attention_recurrence_step_amd", "csrc", "*")):
        text = open(path).read()
        assert "getenv" not in text and "environ" not in text, path
