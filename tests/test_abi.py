"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, the header is plain C, struct layouts agree with the binding,
and configuration / size validation behaves as documented."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

import token_level_gather_amd as kvs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvs.h")


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(kvs_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    lib = kvs.lib()
    declared = _declared_functions()
    assert len(declared) >= 13
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(kvs.EXPORTS) == declared


def test_checked_build_exports_every_declared_symbol():
    # the device-checked debug build is the same C ABI
    lib = kvs.load_library(kvs.CHECKED_LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert lib.kvs_strerror(kvs.KVS_EBOUNDS).decode() == kvs.strerror(kvs.KVS_EBOUNDS)
    assert lib is not kvs.lib()


def test_binding_constants_match_header():
    # every integer #define of the header that the binding also names
    text = open(HEADER).read()
    defines = dict(re.findall(r"^#define\s+(KVS_\w+)\s+\(?(-?\d+)\)?", text, re.M))
    named = [n for n in defines if hasattr(kvs, n)]
    assert {"KVS_EBOUNDS", "KVS_ECORRUPT", "KVS_SITE_LRU_ORDER", "KVS_SITE_APPEND",
            "KVS_FLAG_CHECK", "KVS_FLAG_SEPARATE_ATTENTION"} <= set(named)
    for n in named:
        assert getattr(kvs, n) == int(defines[n]), n


def test_header_is_plain_c():
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "t.c")
        with open(src, "w") as f:
            f.write('#include "kvs.h"\nint main(void){kvs_config c; (void)c; return 0;}\n')
        subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER),
                        "-fsyntax-only", src], check=True)


def test_struct_layouts_match_binding():
    structs = {
        "kvs_config": kvs.kvs_config, "kvs_sizes": kvs.kvs_sizes,
        "kvs_buffers": kvs.kvs_buffers, "kvs_step_stats": kvs.kvs_step_stats,
        "kvs_unit_state": kvs.kvs_unit_state, "kvs_kernel_times": kvs.kvs_kernel_times,
    }
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "kvs.h"', "int main(void){"]
    for cname, py in structs.items():
        lines.append(f'printf("{cname} %zu\\n", sizeof({cname}));')
        for field, _ in py._fields_:
            lines.append(f'printf("{cname}.{field} %zu\\n", offsetof({cname}, {field}));')
    lines.append("return 0;}")
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "t.c"), os.path.join(d, "t")
        open(src, "w").write("\n".join(lines))
        subprocess.run(["gcc", "-I", os.path.dirname(HEADER), src, "-o", exe], check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    got = dict(l.split() for l in out.splitlines())
    for cname, py in structs.items():
        assert int(got[cname]) == ctypes.sizeof(py), cname
        for field, _ in py._fields_:
            assert int(got[f"{cname}.{field}"]) == getattr(py, field).offset, (cname, field)


def test_query_sizes_arithmetic():
    cfg = kvs.make_config(batch=64, layers=1, context=16384, slots=4096, topk=2048)
    s = kvs.query_sizes(cfg)
    assert s.host_pool_bytes == 64 * 16384 * 1152 == 1_207_959_552
    assert s.hot_bytes == 64 * 4096 * 1152 == 301_989_888
    assert s.cbuf_bytes == 64 * 2048 * 1152 == 150_994_944
    # maps: tok2slot + slot2tok + last_used + order (+ small counters)
    assert s.meta_bytes >= 64 * (16384 * 4 + 4096 * 10)
    assert s.meta_bytes < 64 * (16384 * 4 + 4096 * 10) + 64 * 64 + 4096
    # assembling launch (default): 128 hit and 128 fetch workgroups in all, so
    # 2 of each per request and 4 partials per request
    assert s.attn_splits == 2 and s.fetch_blocks == 128
    # slot_of, miss_pos, victims, evicted, row_slot, hit_pos, hit_slot,
    # miss_tok [B][K] int32; counts; partials
    per = 8 * 64 * 2048 * 4 + 64 * 16 + 64 * 4 * 16 * (512 + 2) * 4
    assert per <= s.scratch_bytes < per + 12 * 256
    sep = kvs.query_sizes(kvs.make_config(batch=64, layers=1, context=16384, slots=4096,
                                          topk=2048, flags=kvs.KVS_FLAG_SEPARATE_ATTENTION))
    assert sep.attn_splits == 4 and sep.fetch_blocks == 256   # the separate path's split fit
    assert per <= sep.scratch_bytes < per + 12 * 256
    d = kvs.query_sizes(kvs.make_config(batch=64, layers=1, context=16384, slots=4096,
                                        topk=2048, flags=kvs.KVS_FLAG_DIRECT_HOT))
    assert d.cbuf_bytes == 0 and d.hot_bytes == s.hot_bytes


@pytest.mark.parametrize("bad", [
    dict(batch=0), dict(layers=0), dict(topk=0), dict(slots=100, topk=200),
    dict(context=100, topk=200, slots=300), dict(slots=16385), dict(topk=8193, slots=9000),
    dict(heads=8), dict(head_dim=512), dict(v_dim=576), dict(scale=0.0),
    dict(scale=float("inf")), dict(attn_splits=65), dict(flags=32), dict(context=2**31),
    dict(fetch_blocks=-1), dict(fetch_blocks=65536), dict(hit_blocks=-1), dict(hit_blocks=70000),
    dict(attn_splits=33),   # more splits than 64-token tiles (K = 2048 -> 32)
])
def test_bad_configs_rejected(bad):
    args = dict(batch=2, layers=1, context=4096, slots=4096, topk=2048)
    args.update(bad)
    cfg = kvs.make_config(**args)
    out = kvs.kvs_sizes()
    assert kvs.lib().kvs_query_sizes(ctypes.byref(cfg), ctypes.byref(out)) == kvs.KVS_EINVAL


def test_good_config_accepted():
    cfg = kvs.make_config(batch=2, layers=1, context=4096, slots=4096, topk=2048)
    out = kvs.kvs_sizes()
    assert kvs.lib().kvs_query_sizes(ctypes.byref(cfg), ctypes.byref(out)) == kvs.KVS_OK


def test_create_pool_argument_checks_before_any_gpu_call():
    lib = kvs.lib()
    cfg = kvs.make_config(batch=1, layers=1, context=4096, slots=512, topk=256)
    handle = ctypes.c_void_p()
    rc = lib.kvs_create_pool(ctypes.byref(cfg), None, None, ctypes.byref(handle))
    assert rc == kvs.KVS_EINVAL
    fake = 1 << 20   # aligned, never dereferenced: the size check fails first
    bufs = kvs.kvs_buffers(fake, fake, fake, fake, fake, 16, 16, 16, 16, 16)
    assert lib.kvs_create_pool(ctypes.byref(cfg), ctypes.byref(bufs), None,
                               ctypes.byref(handle)) == kvs.KVS_ENOMEM
    nul = kvs.kvs_buffers(None, fake, fake, fake, fake, 1 << 40, 1 << 40, 1 << 40, 1 << 40, 1 << 40)
    assert lib.kvs_create_pool(ctypes.byref(cfg), ctypes.byref(nul), None,
                               ctypes.byref(handle)) == kvs.KVS_EINVAL
    assert handle.value is None


def test_null_pool_calls_are_rejected():
    lib = kvs.lib()
    assert lib.kvs_step(None, 0, None, None, None, None, None) == kvs.KVS_EINVAL
    assert lib.kvs_free_request(None, 0, None) == kvs.KVS_EINVAL
    assert lib.kvs_release(None) == kvs.KVS_EINVAL
    assert lib.kvs_publish(None, 0, 0, 0, 0, None) == kvs.KVS_EINVAL
    assert lib.kvs_publish_device(None, 0, 0, 0, 0, None, None) == kvs.KVS_EINVAL
    assert lib.kvs_append(None, 0, None, None, None) == kvs.KVS_EINVAL
    assert lib.kvs_probe_host_read(None, 0, None, None) == kvs.KVS_EINVAL
    assert lib.kvs_probe_host_read(None, 16, None, None) == kvs.KVS_EINVAL
    assert lib.kvs_probe_hit_copy(None, 0, None) == kvs.KVS_EINVAL
    assert lib.kvs_profile_begin(None, 1, 1) == kvs.KVS_EINVAL


def test_padded_flag_accepted():
    cfg = kvs.make_config(batch=2, layers=1, context=4096, slots=512, topk=256,
                          flags=kvs.KVS_FLAG_PADDED_TOPK | kvs.KVS_FLAG_HITS_FIRST
                          | kvs.KVS_FLAG_DIRECT_HOT | kvs.KVS_FLAG_CHECK
                          | kvs.KVS_FLAG_SEPARATE_ATTENTION)
    out = kvs.kvs_sizes()
    assert kvs.lib().kvs_query_sizes(ctypes.byref(cfg), ctypes.byref(out)) == kvs.KVS_OK


def test_strerror():
    assert "state check" in kvs.strerror(kvs.KVS_ECORRUPT)
    assert "duplicate" in kvs.strerror(kvs.KVS_EDUP)
    assert "outside" in kvs.strerror(kvs.KVS_ERANGE)
    assert kvs.strerror(kvs.KVS_OK) == "ok"
    assert "HIP" in kvs.strerror(kvs.KVS_EHIP_BASE - 2)
    assert "bounds" in kvs.strerror(kvs.KVS_EBOUNDS)


def test_fetch_blocks_resolve():
    s = kvs.query_sizes(kvs.make_config(batch=64, layers=1, context=16384, slots=4096, topk=2048))
    assert s.fetch_blocks == 128
    s = kvs.query_sizes(kvs.make_config(batch=64, layers=1, context=16384, slots=4096, topk=2048,
                                        fetch_blocks=300))
    assert s.fetch_blocks == 300
    s = kvs.query_sizes(kvs.make_config(batch=64, layers=1, context=16384, slots=4096, topk=2048,
                                        flags=kvs.KVS_FLAG_SEPARATE_ATTENTION))
    assert s.fetch_blocks == 256


def _separate_parts(batch, topk):
    """Partials per request of the separate attention: its workgroups share the
    batch * ceil(topk/64) tiles evenly (one round of at most 256, the fewest
    that reach ceil(tiles / 256) each); a request's partials are the
    workgroups its tiles fall in."""
    t = -(-topk // 64)
    g = batch * t
    per = -(-g // 256)
    w = -(-g // per)

    def share(tile):   # workgroup whose share [w*g//W, (w+1)*g//W) holds the tile
        return next(i for i in range(w) if i * g // w <= tile < (i + 1) * g // w)
    return max(share(b * t + t - 1) - share(b * t) + 1 for b in range(batch))


@pytest.mark.parametrize("batch,topk,parts", [
    (192, 2048, 2), (64, 2048, 4), (32, 2048, 8), (4, 2048, 32), (1, 256, 4), (17, 2048, 12),
    (9, 2100, 17)])
def test_separate_attention_partials(batch, topk, parts):
    s = kvs.query_sizes(kvs.make_config(batch=batch, layers=1, context=max(4096, topk),
                                        slots=topk, topk=topk,
                                        flags=kvs.KVS_FLAG_SEPARATE_ATTENTION))
    assert s.attn_splits == parts == _separate_parts(batch, topk)


@pytest.mark.parametrize("batch,topk,hit_splits,fetch_blocks", [
    (1, 256, 4, 64),      # 8 hit workgroups wanted, but only 4 tiles of 64
    (4, 2048, 8, 64),     # at most 8 per request; at least 64 fetch workgroups
    (32, 2048, 4, 96),    # three fetch workgroups per request
    (48, 2048, 3, 128),
    (64, 2048, 2, 128),
    (192, 2048, 1, 128),  # at most 128 fetch workgroups (still one per request)
    (3, 8192, 8, 64),
])
def test_default_assemble_counts(batch, topk, hit_splits, fetch_blocks):
    s = kvs.query_sizes(kvs.make_config(batch=batch, layers=1, context=20000, slots=topk,
                                        topk=topk))
    assert s.attn_splits == hit_splits and s.fetch_blocks == fetch_blocks


def test_graph_calls_reject_null():
    lib = kvs.lib()
    g = ctypes.c_void_p()
    assert lib.kvs_graph_capture(None, 0, None, None, None, None, ctypes.byref(g)) == kvs.KVS_EINVAL
    assert lib.kvs_graph_launch(None, None) == kvs.KVS_EINVAL
    assert lib.kvs_graph_destroy(None) == kvs.KVS_EINVAL
