"""Host-side checks of the C-ABI that need no GPU: the library loads, exports
every function include/ls.h declares, sizes workspaces, and rejects bad
arguments before anything is enqueued (so no HIP call is made)."""
import ctypes
import subprocess

import pytest
import torch

import top_sparse_attention_ls_amd as ls


@pytest.fixture(scope="module")
def lib():
    return ls.load()


def test_exports_every_declared_function(lib):
    names = ls.header_symbols()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", ls.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    assert set(names) <= exported


def test_header_compiles_as_c99(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "ls.h"\nint main(void){ return ls_abi_version() == 0; }\n')
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-c", "-I",
                        ls.HEADER_PATH.rsplit("/", 1)[0], str(src), "-o", str(tmp_path / "t.o")],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_struct_layouts_match_header(tmp_path):
    src = tmp_path / "s.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "ls.h"\n'
                   'int main(void){ printf("%zu %zu %zu %zu %zu %zu %zu %zu\\n",'
                   ' sizeof(ls_idx_desc), sizeof(ls_hot_desc), sizeof(ls_attn_desc),'
                   ' sizeof(ls_step_desc), sizeof(ls_step_io), sizeof(ls_prefill_desc),'
                   ' offsetof(ls_attn_desc, scale), offsetof(ls_step_desc, attn));'
                   ' printf("%zu %zu %zu\\n", sizeof(ls_commit_desc), sizeof(ls_append_desc),'
                   ' offsetof(ls_step_desc, commit)); return 0; }\n')
    exe = tmp_path / "s"
    subprocess.check_call(["gcc", "-std=c99", "-I", ls.HEADER_PATH.rsplit("/", 1)[0], str(src),
                           "-o", str(exe)])
    got = [int(x) for x in subprocess.check_output([str(exe)]).split()]
    want = [ctypes.sizeof(ls.IdxDesc), ctypes.sizeof(ls.HotDesc), ctypes.sizeof(ls.AttnDesc),
            ctypes.sizeof(ls.StepDesc), ctypes.sizeof(ls.StepIO), ctypes.sizeof(ls.PrefillDesc),
            ls.AttnDesc.scale.offset, ls.StepDesc.attn.offset, ctypes.sizeof(ls.CommitDesc),
            ctypes.sizeof(ls.AppendDesc), ls.StepDesc.commit.offset]
    assert got == want


def test_version_and_error_string(lib):
    assert lib.ls_abi_version() == ls.ABI_VERSION == 5
    assert isinstance(lib.ls_last_error(), bytes)


def idx(**kw):
    base = dict(batch=2, max_ctx=4096, n_heads=64, head_dim=128, n_cand=1024, topk=256)
    base.update(kw)
    return ls.IdxDesc(**base)


def test_workspace_sizes(lib):
    n = lib.ls_workspace_size(ls.OP_COARSE, ctypes.byref(idx()))
    # scores + two tie arrays dominate: 3 * B * L * 4 bytes
    assert n >= 3 * 2 * 4096 * 4
    assert lib.ls_workspace_size(ls.OP_REFINE, ctypes.byref(idx())) >= 2 * 1024 * 8
    bad = idx(head_dim=96)
    assert lib.ls_workspace_size(ls.OP_COARSE, ctypes.byref(bad)) == 0
    assert b"head_dim" in lib.ls_last_error()
    assert lib.ls_workspace_size(99, ctypes.byref(idx())) == 0


def test_step_workspace_grows_with_batch(lib):
    def step(b):
        i = idx(batch=b, max_ctx=131072, n_cand=8192, topk=2048)
        h = ls.HotDesc(b, 131072, 2048, 4096, 576, 0)
        a = ls.AttnDesc(b, 128, 1, 576, 512, 2048, 4096 + 2048, 576, 0, 0.07, 0)
        return lib.ls_workspace_size(ls.OP_STEP, ctypes.byref(ls.StepDesc(i, h, a, 1)))
    assert 0 < step(1) < step(32)


FAKE = ctypes.c_void_p(0x100000)   # aligned, never dereferenced: validation fails first


@pytest.mark.parametrize("kw,code,needle", [
    (dict(batch=0), ls.LS_E_ARG, b"batch"),
    (dict(max_ctx=0), ls.LS_E_ARG, b"max_ctx"),
    (dict(n_cand=0), ls.LS_E_ARG, b"n_cand"),
    (dict(topk=0), ls.LS_E_ARG, b"topk"),
    (dict(n_heads=65), ls.LS_E_UNSUPPORTED, b"n_heads"),
    (dict(head_dim=32), ls.LS_E_UNSUPPORTED, b"head_dim"),
])
def test_index_coarse_rejects_bad_shapes(lib, kw, code, needle):
    d = idx(**kw)
    rc = lib.ls_index_coarse(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert rc == code
    assert needle in lib.ls_last_error()


def test_null_pointers_rejected(lib):
    d = idx()
    rc = lib.ls_index_coarse(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert rc == ls.LS_E_ARG and b"null" in lib.ls_last_error()
    rc = lib.ls_refine_topk(ctypes.byref(d), FAKE, FAKE, FAKE, None, None, None, FAKE, FAKE,
                            None, FAKE, 1 << 30, None)
    assert rc == ls.LS_E_ARG


@pytest.mark.parametrize("kw,kp,kc,needle", [
    (dict(keys_on_host=2), None, None, b"keys_on_host"),
    (dict(key_slots=-1), None, None, b"key_slots"),
    (dict(key_slots=(1 << 24) + 1), FAKE, FAKE, b"key_slots"),
    (dict(key_slots=1024), None, FAKE, b"kpos2slot"),
    (dict(key_slots=1024), FAKE, None, b"kcache"),
    (dict(key_slots=1024), FAKE, ctypes.c_void_p(0x100008), b"aligned"),
])
def test_refine_key_source_validated(lib, kw, kp, kc, needle):
    # the key source is checked on the host before any launch (and before
    # any pointer query), whatever the key cache and host-key flags say
    d = idx(**kw)
    rc = lib.ls_refine_topk(ctypes.byref(d), FAKE, FAKE, FAKE, kp, kc, FAKE, FAKE, FAKE, None,
                            FAKE, 1 << 30, None)
    assert rc == ls.LS_E_ARG
    assert needle in lib.ls_last_error()


def test_misaligned_rejected(lib):
    d = idx()
    rc = lib.ls_index_coarse(ctypes.byref(d), FAKE, FAKE, ctypes.c_void_p(0x100001), FAKE, FAKE,
                             FAKE, 1 << 30, None)
    assert rc == ls.LS_E_ARG and b"aligned" in lib.ls_last_error()


def test_workspace_too_small_rejected(lib):
    d = idx()
    rc = lib.ls_index_coarse(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1024, None)
    assert rc == ls.LS_E_WORKSPACE and b"too small" in lib.ls_last_error()
    rc = lib.ls_index_coarse(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, 1 << 30, None)
    assert rc == ls.LS_E_WORKSPACE


def test_attention_validation(lib):
    a = ls.AttnDesc(2, 12, 5, 64, 64, 16, 100, 320, 64, 0.125, 0)   # 12 % 5 != 0
    rc = lib.ls_sparse_attn_decode(ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   1 << 30, None)
    assert rc == ls.LS_E_ARG and b"multiple" in lib.ls_last_error()
    a = ls.AttnDesc(2, 8, 8, 64, 64, 16, 100, 512, 64, float("nan"), 0)
    rc = lib.ls_sparse_attn_decode(ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   1 << 30, None)
    assert rc == ls.LS_E_ARG and b"finite" in lib.ls_last_error()
    a = ls.AttnDesc(2, 8, 8, 2048, 64, 16, 100, 512, 64, 0.1, 0)
    rc = lib.ls_sparse_attn_decode(ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   1 << 30, None)
    assert rc == ls.LS_E_UNSUPPORTED
    # the generic kernel reads 16-byte pieces: a row stride off the 8-element grid is refused
    a = ls.AttnDesc(2, 8, 8, 64, 64, 16, 100, 516, 64, 0.1, 0)
    rc = lib.ls_sparse_attn_decode(ctypes.byref(a), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   1 << 30, None)
    assert rc == ls.LS_E_UNSUPPORTED and b"multiples of 8" in lib.ls_last_error()


def test_step_validation(lib):
    i = idx()
    h = ls.HotDesc(2, 4096, 256, 64, 576, 0)
    a = ls.AttnDesc(2, 128, 1, 576, 512, 256, 64 + 256, 576, 0, 0.07, 0)
    io = ls.StepIO()
    rc = lib.ls_decode_step(ctypes.byref(ls.StepDesc(i, h, a, 1)), ctypes.byref(io), FAKE,
                            1 << 30, None)
    assert rc == ls.LS_E_ARG and b"null" in lib.ls_last_error()
    a_bad = ls.AttnDesc(3, 128, 1, 576, 512, 256, 64 + 256, 576, 0, 0.07, 0)
    rc = lib.ls_decode_step(ctypes.byref(ls.StepDesc(i, h, a_bad, 1)), ctypes.byref(io), FAKE,
                            1 << 30, None)
    assert rc == ls.LS_E_ARG and b"match" in lib.ls_last_error()
    rc = lib.ls_decode_step(None, ctypes.byref(io), FAKE, 1 << 30, None)
    assert rc == ls.LS_E_ARG


def test_pack_validation(lib):
    assert lib.ls_pack_coarse(FAKE, FAKE, 10, 6, None) == ls.LS_E_ARG
    assert lib.ls_pack_coarse(None, FAKE, 10, 8, None) == ls.LS_E_ARG
    assert lib.ls_pack_coarse(FAKE, FAKE, -1, 8, None) == ls.LS_E_ARG
    assert lib.ls_pack_coarse(FAKE, FAKE, 0, 8, None) == ls.LS_OK   # nothing to do


def test_python_binding_requires_gpu_tensors_types():
    import torch
    with pytest.raises(TypeError):
        ls.pack_coarse(torch.zeros(4, 8, dtype=torch.uint8))


def test_binding_rejects_mis_sized_tensors():
    """The library trusts the descriptor's sizes; the binding checks every
    tensor against them before a launch (a short hot buffer would otherwise
    be written past its end)."""
    import torch
    import top_sparse_attention_ls_amd as ls
    t = torch.zeros((2, 5, 8), dtype=torch.bfloat16)
    ls._need(t, torch.bfloat16, "hot", (2, 5, 8))
    with pytest.raises(ValueError):
        ls._need(t, torch.bfloat16, "hot", (2, 6, 8))
    with pytest.raises(TypeError):
        ls._need(t, torch.float32, "hot", (2, 5, 8))
    with pytest.raises(ValueError):
        ls._need(t.transpose(1, 2), torch.bfloat16, "hot")
    with pytest.raises(ValueError):
        ls._need_rows(t, 81, "k_base")


@pytest.mark.parametrize("args,needle", [
    (dict(n_slots=0), b"slots"),
    (dict(n_slots=16385), b"slots"),
    (dict(n=0), b"entries"),
    (dict(n=16385), b"entries"),
    (dict(now=0xFFFFFFFF), b"now"),
    (dict(batch=0), b"batch"),
])
def test_cache_commit_rejects_bad_shapes(lib, args, needle):
    a = dict(batch=2, max_ctx=4096, n_slots=1024, n=256, now=5)
    a.update(args)
    rc = lib.ls_cache_commit(a["batch"], a["max_ctx"], a["n_slots"], a["n"], a["now"], FAKE,
                             FAKE, FAKE, FAKE, FAKE, None, None)
    assert rc == ls.LS_E_ARG
    assert needle in lib.ls_last_error()


def test_cache_commit_null_table_rejected(lib):
    rc = lib.ls_cache_commit(2, 4096, 1024, 256, 5, FAKE, FAKE, None, FAKE, FAKE, None, None)
    assert rc == ls.LS_E_ARG and b"slot2pos" in lib.ls_last_error()


@pytest.mark.parametrize("kw,needle", [
    (dict(head_dim=96), b"head_dim"),
    (dict(row_elems=12), b"row_elems"),
    (dict(keys_on_host=3), b"keys_on_host"),
    (dict(row_elems=576), b"new_kv"),
])
def test_append_rejects_bad_arguments(lib, kw, needle):
    base = dict(batch=2, max_ctx=4096, head_dim=128, row_elems=0, keys_on_host=0, pool_on_host=0)
    base.update(kw)
    d = ls.AppendDesc(**base)
    rc = lib.ls_append_token(ctypes.byref(d), FAKE, None, FAKE, FAKE, None, FAKE, None)
    assert rc in (ls.LS_E_ARG, ls.LS_E_UNSUPPORTED)
    assert needle in lib.ls_last_error()


def step_desc(commit_hot=0, commit_keys=0, key_slots=0, now=1, hot_slots=4096):
    i = idx(batch=2, max_ctx=131072, n_cand=8192, topk=2048, key_slots=key_slots)
    h = ls.HotDesc(2, 131072, 2048, hot_slots, 576, 0)
    a = ls.AttnDesc(2, 128, 1, 576, 512, 2048, hot_slots + 2048, 576, 0, 0.07, 0)
    return ls.StepDesc(i, h, a, 1, ls.CommitDesc(commit_hot, commit_keys, now))


def fake_io(**kw):
    io = ls.StepIO()
    for name, _ in ls.StepIO._fields_:
        setattr(io, name, 0x100000)
    io.stage_events = None
    for k, v in kw.items():
        setattr(io, k, v)
    return io


@pytest.mark.parametrize("desc,io_kw,needle", [
    (dict(commit_keys=1), {}, b"key_slots"),
    (dict(commit_hot=1, hot_slots=20000), {}, b"slots"),
    (dict(commit_hot=1, now=0xFFFFFFFF), {}, b"now"),
    (dict(commit_hot=1), dict(stamp_dev=None), b"stamp"),
    (dict(commit_keys=1, key_slots=16384), dict(kslot2pos_dev=None), b"kslot2pos"),
    (dict(commit_hot=2), {}, b"commit"),
])
def test_step_commit_validated(lib, desc, io_kw, needle):
    d = step_desc(**desc)
    rc = lib.ls_decode_step(ctypes.byref(d), ctypes.byref(fake_io(**io_kw)), FAKE, 1 << 40, None)
    assert rc == ls.LS_E_ARG
    assert needle in lib.ls_last_error()


def test_binding_checks_key_cache_and_append_arguments():
    # argument checks of the binding run before anything touches a device
    q = torch.zeros((2, 4, 64), dtype=torch.int8)
    w = torch.zeros((2, 4), dtype=torch.int8)
    k8 = torch.zeros((2, 100, 64), dtype=torch.int8)
    cand = torch.zeros((2, 16), dtype=torch.int32)
    cl = torch.zeros((2,), dtype=torch.int32)
    with pytest.raises(ValueError, match="go together"):
        ls.refine_topk(q, w, k8, cand, cl, 8, kpos2slot=torch.zeros((2, 100), dtype=torch.int32))
    with pytest.raises(ValueError, match="kpos2slot"):
        ls.refine_topk(q, w, k8, cand, cl, 8, kpos2slot=torch.zeros((2, 99), dtype=torch.int32),
                       kcache=torch.zeros((2, 10, 64), dtype=torch.int8))
    with pytest.raises(ValueError, match="device memory"):
        ls.refine_topk(q, w, k8, cand, cl, 8, kpos2slot=torch.zeros((2, 100), dtype=torch.int32),
                       kcache=torch.zeros((2, 10, 64), dtype=torch.int8))
    kc = torch.zeros((2, 100, 32), dtype=torch.uint8)
    with pytest.raises(ValueError, match="go together"):
        ls.append_token(torch.zeros((2, 64), dtype=torch.int8), k8, kc, cl,
                        new_kv=torch.zeros((2, 576), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="kc"):
        ls.append_token(torch.zeros((2, 64), dtype=torch.int8), k8, kc[:, :, :16].contiguous(), cl)


def test_shapes_whose_32_bit_offsets_would_wrap_are_rejected(lib):
    # the miss gather addresses a request's miss rows, and the prefill
    # scoring the key history, with 32-bit byte offsets: shapes beyond them
    # are refused before any launch instead of wrapping
    h = ls.HotDesc(2, 4096, 1 << 20, 64, 2048, 0)          # 2^20 * 2048 * 2 = 2^32 bytes
    rc = lib.ls_hot_gather(ctypes.byref(h), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30,
                           None)
    assert rc == ls.LS_E_UNSUPPORTED and b"2^32" in lib.ls_last_error()
    p = ls.PrefillDesc(16, (1 << 24) + 8, 0, 64, 128, 64)   # max_ctx * 128 > 2^31
    rc = lib.ls_prefill_index_topk(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert rc == ls.LS_E_UNSUPPORTED and b"2^31" in lib.ls_last_error()
    p = ls.PrefillDesc(16, 1 << 23, 0, 64, 128, 64)         # 2^30: accepted by the shape check
    assert lib.ls_workspace_size(ls.OP_PREFILL, ctypes.byref(p)) > 0


def test_read_probe_validation(lib):
    # measurement helper: checked on the host like every entry point
    assert lib.ls_read_probe(None, 1024, None, 0, 0, FAKE, None) == ls.LS_E_ARG
    assert lib.ls_read_probe(FAKE, 1000, None, 0, 0, FAKE, None) == ls.LS_E_ARG
    assert b"multiple of 16" in lib.ls_last_error()
    assert lib.ls_read_probe(FAKE, 1024, FAKE, 4, 100, FAKE, None) == ls.LS_E_ARG
    assert lib.ls_read_probe(FAKE, 1024, FAKE, 4, 2048, FAKE, None) == ls.LS_E_ARG
    assert b"whole row" in lib.ls_last_error()
    assert lib.ls_read_probe(FAKE, 1024, FAKE, 4, 256, FAKE, None) == ls.LS_E_UNSUPPORTED
    assert lib.ls_read_probe(FAKE, 1024, None, 0, 0, None, None) == ls.LS_E_ARG


def test_noalloc_step_checks_its_scratch_limit_before_the_device(lib):
    # ls_decode_step_noalloc refuses a step whose workspace exceeds its static
    # scratch, and a null descriptor, before any device call
    assert lib.ls_decode_step_noalloc(None, FAKE, None) == ls.LS_E_ARG
    i = idx(batch=64, max_ctx=131072, n_cand=8192, topk=2048)
    h = ls.HotDesc(64, 131072, 2048, 4096, 576, 0)
    a = ls.AttnDesc(64, 128, 1, 576, 512, 2048, 4096 + 2048, 576, 0, 0.07, 0)
    d = ls.StepDesc(i, h, a, 1)
    assert lib.ls_workspace_size(ls.OP_STEP, ctypes.byref(d)) > 128 << 20
    rc = lib.ls_decode_step_noalloc(ctypes.byref(d), ctypes.byref(ls.StepIO()), None)
    assert rc == ls.LS_E_UNSUPPORTED and b"static scratch" in lib.ls_last_error()
