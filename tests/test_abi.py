"""The C-ABI library loads, exports what include/pkv.h declares, and rejects
bad host-side arguments with the documented status before any launch (no GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

from paged_kv_cache_prepare_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\S.*?\b(pkv_[a-z0-9_]+)\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return binding.load()


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(binding.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (pkv_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_status_strings(lib):
    for code in range(7):
        assert binding.status_string(code) != "unknown status"
    assert binding.status_string(99) == "unknown status"


def test_checked_build_exports_the_same_symbols():
    out = subprocess.run(["nm", "-D", "--defined-only", binding.CHECKED_LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (pkv_\w+)", out))
    assert set(declared_functions()) <= exported
    regular = ctypes.CDLL(binding.REGULAR_LIB_PATH)
    checked = ctypes.CDLL(binding.CHECKED_LIB_PATH)
    assert regular.pkv_debug_checks_enabled() == 0
    assert checked.pkv_debug_checks_enabled() == 1
    # the checked build keeps the flags of this process's last failed check
    assert regular.pkv_debug_check_flags() == 0


def test_check_bits_match_the_header():
    text = open(HEADER).read()
    bits = {m.group(1).lower(): int(m.group(2), 16)
            for m in re.finditer(r"#define PKV_CHECK_(\w+) (0x[0-9a-f]+)u", text)}
    assert bits == binding.CHECK_BITS


def test_checked_build_validates_host_arguments_first():
    checked = binding.use_checked(True)
    try:
        # host-side rejections come before any device-side check (no GPU needed)
        assert kvw(checked, T=-1) == binding.ERR_INVALID_ARG
        assert attn(checked, Hq=6, Hkv=4) == binding.ERR_INVALID_ARG
        assert block_op(checked, "pkv_zero_blocks", bb=1000) == binding.ERR_UNSUPPORTED
        assert kvw(checked, T=0, k=None, v=None, slot=None) == binding.OK
    finally:
        binding.use_checked(False)


FAKE = 0x10000  # aligned, never dereferenced: every call below returns before launching


def prep(lib, **kw):
    a = dict(nst=FAKE, nct=FAKE, bt=FAKE, stride=4, R=3, T=10, qsl_len=4, bs=16, nb=16,
             ri=FAKE, pos=FAKE, slot=FAKE, qsl=FAKE, sl=FAKE, li=FAKE)
    a.update(kw)
    return lib.pkv_prepare_inputs(a["nst"], a["nct"], a["bt"], a["stride"], a["R"], a["T"],
                                  a["qsl_len"], a["bs"], a["nb"], a["ri"], a["pos"], a["slot"],
                                  a["qsl"], a["sl"], a["li"], None)


@pytest.mark.parametrize("kw", [dict(R=-1), dict(T=-1), dict(qsl_len=3), dict(bs=0),
                                dict(nb=-1), dict(qsl=None), dict(nst=None), dict(bt=None),
                                dict(slot=None), dict(stride=0), dict(R=0, qsl_len=1)])
def test_prepare_rejects(lib, kw):
    assert prep(lib, **kw) == binding.ERR_INVALID_ARG


def kvw(lib, **kw):
    a = dict(k=FAKE, v=FAKE, ks=256, vs=256, kc=FAKE, vc=FAKE, nb=8, slot=FAKE, T=4, H=2, d=128,
             bs=16, dt=binding.BF16)
    a.update(kw)
    return lib.pkv_kv_cache_write(a["k"], a["v"], a["ks"], a["vs"], a["kc"], a["vc"], a["nb"],
                                  a["slot"], a["T"], a["H"], a["d"], a["bs"], a["dt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), binding.ERR_INVALID_ARG), (dict(H=0), binding.ERR_INVALID_ARG),
    (dict(bs=0), binding.ERR_INVALID_ARG), (dict(dt=7), binding.ERR_INVALID_ARG),
    (dict(k=None), binding.ERR_INVALID_ARG), (dict(ks=255), binding.ERR_INVALID_ARG),
    (dict(k=FAKE + 2), binding.ERR_INVALID_ARG), (dict(d=100), binding.ERR_UNSUPPORTED),
    (dict(d=512), binding.ERR_UNSUPPORTED)])
def test_kv_write_rejects(lib, kw, code):
    assert kvw(lib, **kw) == code


def test_kv_write_empty_is_ok(lib):
    assert kvw(lib, T=0, k=None, v=None, slot=None) == binding.OK


def attn(lib, **kw):
    a = dict(q=FAKE, qs=4 * 128, kc=FAKE, vc=FAKE, nb=16, out=FAKE, os=4 * 128, qsl=FAKE,
             sl=FAKE, bt=FAKE, bts=8, R=3, T=10, mq=5, ms=100, Hq=4, Hkv=2, d=128, bs=16,
             scale=0.1, dt=binding.BF16, split=0, ws=None, wsb=0)
    a.update(kw)
    return lib.pkv_paged_attention_varlen(
        a["q"], a["qs"], a["kc"], a["vc"], a["nb"], a["out"], a["os"], a["qsl"], a["sl"],
        a["bt"], a["bts"], a["R"], a["T"], a["mq"], a["ms"], a["Hq"], a["Hkv"], a["d"], a["bs"],
        a["scale"], a["dt"], a["split"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(Hq=6, Hkv=4), binding.ERR_INVALID_ARG), (dict(R=-1), binding.ERR_INVALID_ARG),
    (dict(split=48), binding.ERR_INVALID_ARG), (dict(split=-32), binding.ERR_INVALID_ARG),
    (dict(dt=3), binding.ERR_INVALID_ARG), (dict(d=96), binding.ERR_UNSUPPORTED),
    (dict(scale=0.0), binding.ERR_INVALID_ARG), (dict(scale=-0.1), binding.ERR_INVALID_ARG),
    (dict(scale=float("nan")), binding.ERR_INVALID_ARG),
    (dict(scale=float("inf")), binding.ERR_INVALID_ARG),
    (dict(bs=32), binding.ERR_UNSUPPORTED), (dict(Hq=64, Hkv=2), binding.ERR_UNSUPPORTED),
    (dict(q=None), binding.ERR_INVALID_ARG), (dict(qs=100), binding.ERR_INVALID_ARG),
    (dict(out=FAKE + 8), binding.ERR_INVALID_ARG), (dict(bts=0), binding.ERR_INVALID_ARG),
    (dict(), binding.ERR_WORKSPACE), (dict(ws=FAKE, wsb=16), binding.ERR_WORKSPACE),
    (dict(ws=FAKE + 16, wsb=1 << 30), binding.ERR_WORKSPACE)])
def test_attention_rejects(lib, kw, code):
    assert attn(lib, **kw) == code


def test_attention_empty_batch_is_ok(lib):
    assert attn(lib, T=0, R=0, q=None, out=None, qsl=None, sl=None, bt=None) == binding.OK


def test_workspace_sizes():
    ws = binding.attention_workspace_bytes
    assert ws(3, 10, 4, 2, 128, 5, 100) > 0
    assert ws(3, 10, 6, 4, 128, 5, 100) == 0                     # Hq % Hkv != 0
    import torch
    assert ws(3, 10, 4, 2, 64, 5, 100, dtype=torch.float32) == 0   # fp32 path needs none
    # forcing partitions adds partial-result storage
    assert ws(16, 16, 64, 8, 128, 1, 32768, split_tokens=1024) > ws(16, 16, 64, 8, 128, 1, 32768,
                                                                    split_tokens=32768)
    # one request with more query rows than a decode tile: no partitions, so
    # the workspace holds only the work list (the default for two such
    # requests, which may hide a decode, partitions the contexts)
    one = ws(1, 5000, 32, 8, 128, 5000, 8000)
    assert one == ws(1, 5000, 32, 8, 128, 5000, 8000, split_tokens=8000)
    assert ws(2, 5000, 32, 8, 128, 5000, 8000) > ws(2, 5000, 32, 8, 128, 5000, 8000,
                                                    split_tokens=8000)
    # one request of 4 rows at G = 4 is a decode item: partitions as before
    assert ws(1, 4, 32, 8, 128, 4, 8000) > ws(1, 4, 32, 8, 128, 4, 8000, split_tokens=8000)
    # every configuration's workspace is modest next to HBM
    assert ws(17, 2064, 64, 8, 128, 2048, 32768) < (256 << 20)
    assert ws(201, 5200, 32, 8, 128, 5000, 8192) < (256 << 20)


def input_ids(lib, **kw):
    a = dict(tt=FAKE, M=64, R=3, ri=FAKE, pos=FAKE, T=10, sl=FAKE, tot=FAKE, ti=None, ids=FAKE,
             dm=FAKE)
    a.update(kw)
    return lib.pkv_prepare_input_ids(a["tt"], a["M"], a["R"], a["ri"], a["pos"], a["T"],
                                     a["sl"], a["tot"], a["ti"], a["ids"], a["dm"], None)


@pytest.mark.parametrize("kw", [dict(M=0), dict(R=-1), dict(T=-1), dict(tt=None),
                                dict(ri=None), dict(ids=None), dict(sl=None), dict(tot=None),
                                dict(dm=None)])
def test_input_ids_rejects(lib, kw):
    assert input_ids(lib, **kw) == binding.ERR_INVALID_ARG


def test_input_ids_empty_is_ok(lib):
    assert input_ids(lib, T=0, R=0, tt=None, ri=None, pos=None, sl=None, tot=None, ids=None,
                     dm=None) == binding.OK


def block_op(lib, fn, **kw):
    a = dict(kc=FAKE, vc=FAKE, nb=16, bb=32768, ids=FAKE, n=4)
    a.update(kw)
    return getattr(lib, fn)(a["kc"], a["vc"], a["nb"], a["bb"], a["ids"], a["n"], None)


@pytest.mark.parametrize("fn", ["pkv_copy_blocks", "pkv_zero_blocks"])
@pytest.mark.parametrize("kw,code", [
    (dict(nb=-1), binding.ERR_INVALID_ARG), (dict(bb=8), binding.ERR_INVALID_ARG),
    (dict(n=-1), binding.ERR_INVALID_ARG), (dict(kc=None), binding.ERR_INVALID_ARG),
    (dict(ids=None), binding.ERR_INVALID_ARG), (dict(bb=1000), binding.ERR_UNSUPPORTED),
    (dict(vc=FAKE + 8), binding.ERR_UNSUPPORTED),
    (dict(bb=1 << 30, n=1 << 20), binding.ERR_UNSUPPORTED)])
def test_block_ops_reject(lib, fn, kw, code):
    assert block_op(lib, fn, **kw) == code


@pytest.mark.parametrize("fn", ["pkv_copy_blocks", "pkv_zero_blocks"])
def test_block_ops_empty_is_ok(lib, fn):
    assert block_op(lib, fn, n=0, kc=None, vc=None, ids=None) == binding.OK


def test_attention_rejects_a_work_list_past_the_dispatch_limit(lib):
    # 32-token partitions of 2^30-token contexts: far more than 2^24 - 1 items
    assert attn(lib, R=1000, T=1000, mq=1, ms=1 << 30, split=32) == binding.ERR_UNSUPPORTED


def test_split_tokens_environment_override(monkeypatch):
    args = (16, 16, 64, 8, 128, 1, 32768)
    monkeypatch.delenv("PKV_SPLIT_TOKENS", raising=False)
    forced = binding.attention_workspace_bytes(*args, split_tokens=1024)
    default = binding.attention_workspace_bytes(*args)
    assert forced != default
    monkeypatch.setenv("PKV_SPLIT_TOKENS", "1024")
    assert binding.attention_workspace_bytes(*args) == forced
    assert binding.attention_workspace_bytes(*args, split_tokens=32768) != forced  # argument wins
    assert binding.split_tokens_or_env(0) == 1024 and binding.split_tokens_or_env(64) == 64


def plan(lib, **kw):
    a = dict(qsl=FAKE, sl=FAKE, R=3, T=10, mq=5, ms=100, Hq=4, Hkv=2, d=128, dt=binding.BF16,
             split=0, ws=None, wsb=0)
    a.update(kw)
    return lib.pkv_paged_attention_plan(a["qsl"], a["sl"], a["R"], a["T"], a["mq"], a["ms"],
                                        a["Hq"], a["Hkv"], a["d"], a["dt"], a["split"], a["ws"],
                                        a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(Hq=6, Hkv=4), binding.ERR_INVALID_ARG), (dict(split=48), binding.ERR_INVALID_ARG),
    (dict(d=96), binding.ERR_UNSUPPORTED), (dict(qsl=None), binding.ERR_INVALID_ARG),
    (dict(), binding.ERR_WORKSPACE), (dict(ws=FAKE + 16, wsb=1 << 30), binding.ERR_WORKSPACE)])
def test_plan_rejects(lib, kw, code):
    assert plan(lib, **kw) == code


def test_plan_without_work_is_ok(lib):
    assert plan(lib, T=0, R=0, qsl=None, sl=None) == binding.OK
    assert plan(lib, dt=binding.F32) == binding.OK   # the fp32 path keeps no work list


def run(lib, **kw):
    a = dict(q=FAKE, qs=4 * 128, kc=FAKE, vc=FAKE, nb=16, out=FAKE, os=4 * 128, qsl=FAKE,
             sl=FAKE, bt=FAKE, bts=8, R=3, T=10, mq=5, ms=100, Hq=4, Hkv=2, d=128, bs=16,
             scale=0.1, dt=binding.BF16, ks=None, vs=None, split=0, ws=None, wsb=0)
    a.update(kw)
    return lib.pkv_paged_attention_run(
        a["q"], a["qs"], a["kc"], a["vc"], a["nb"], a["out"], a["os"], a["qsl"], a["sl"],
        a["bt"], a["bts"], a["R"], a["T"], a["mq"], a["ms"], a["Hq"], a["Hkv"], a["d"], a["bs"],
        a["scale"], a["dt"], a["ks"], a["vs"], a["split"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(ks=FAKE), binding.ERR_INVALID_ARG), (dict(ks=FAKE, vs=FAKE, dt=binding.F32),
                                                binding.ERR_INVALID_ARG),
    (dict(bt=None), binding.ERR_INVALID_ARG), (dict(scale=0.0), binding.ERR_INVALID_ARG),
    (dict(bs=32), binding.ERR_UNSUPPORTED), (dict(), binding.ERR_WORKSPACE)])
def test_run_rejects(lib, kw, code):
    assert run(lib, **kw) == code


def test_noalloc_rejects_sizes_beyond_its_scratch(lib):
    """pkv_paged_attention_varlen_noalloc refuses a call whose work list and
    partials exceed PKV_NOALLOC_SCRATCH_BYTES, before any device access."""
    R, Hkv, Hq, d, split, L = 64, 8, 32, 128, 32, 65536
    need = binding.attention_workspace_bytes(R, R, Hq, Hkv, d, 1, L, split)
    assert need > binding.NOALLOC_SCRATCH_BYTES
    text = open(HEADER).read()
    assert "#define PKV_NOALLOC_SCRATCH_BYTES (64u << 20)" in text
    assert binding.NOALLOC_SCRATCH_BYTES == 64 << 20
    st = lib.pkv_paged_attention_varlen_noalloc(FAKE, Hq * d, FAKE, FAKE, 1 << 16, FAKE, Hq * d,
                                                FAKE, FAKE, FAKE, 1 << 12, R, R, 1, L, Hq, Hkv,
                                                d, 16, 0.088, binding.BF16, split, None)
    assert st == binding.ERR_SCRATCH_LIMIT
    # bad host arguments are still reported as such when the sizes fit
    st = lib.pkv_paged_attention_varlen_noalloc(FAKE, Hq * d, FAKE, FAKE, 1 << 16, FAKE, Hq * d,
                                                FAKE, FAKE, FAKE, 1 << 12, 4, 4, 1, 100, 6, 4,
                                                d, 16, 0.088, binding.BF16, 0, None)
    assert st == binding.ERR_INVALID_ARG
