"""The C ABI: the library loads, exports every call include/pagedkv.h declares, and rejects bad
arguments on the host before any launch (CPU; nothing here reaches a GPU)."""
import ctypes as C
import os
import re
import shutil
import subprocess

import pytest

import paged_kv_cache_404_amd as pkv
from paged_kv_cache_404_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedkv.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n.startswith(("pkv_", "paged_"))))


def test_header_declares_the_boundary():
    names = _declared()
    for required in ("paged_cache_append", "paged_attention_decode", "paged_attention_prefill_chunk",
                     "paged_cache_copy_blocks", "pkv_pool_create", "pkv_seq_append", "pkv_build_block_tables",
                     "pkv_build_slot_mapping", "pkv_last_error"):
        assert required in names


def test_every_declared_symbol_is_exported_and_bound():
    names = _declared()
    for n in names:
        assert hasattr(pkv.lib, n), n
    assert sorted(_lib.EXPORTED) == names
    nm = shutil.which("nm")
    if nm:
        out = subprocess.run([nm, "-D", "--defined-only", pkv.LIB_PATH], capture_output=True, text=True).stdout
        syms = set(re.findall(r"\bT\s+(\S+)", out))
        for n in names:
            assert n in syms, n


def test_version_and_error_text():
    assert pkv.version() == 100
    with pytest.raises(pkv.PagedKVError) as e:
        pkv.BlockPool(3, 16, [1, 1, 2])
    assert "permutation" in str(e.value)


NULL = None


def _decode(**kw):
    args = dict(out=1 << 12, out_dtype=pkv.PKV_F32, query=1 << 12, k=1 << 12, v=1 << 12, tables=1 << 12,
                lens=1 << 12, B=4, Hq=32, Hkv=8, D=128, bs=16, max_blocks=8, N=64, max_ctx=128, scale=0.1, ps=0,
                ws=NULL, ws_bytes=0, dtype=pkv.PKV_BF16)
    args.update(kw)
    return pkv.lib.paged_attention_decode(args["out"], args["out_dtype"], args["query"], args["k"], args["v"],
                                          args["tables"], args["lens"], args["B"], args["Hq"], args["Hkv"], args["D"],
                                          args["bs"], args["max_blocks"], args["N"], args["max_ctx"], args["scale"],
                                          args["ps"], args["ws"], args["ws_bytes"], args["dtype"], NULL, NULL)


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=30), pkv.PKV_EINVAL),                 # not a multiple of Hkv
    (dict(bs=32), pkv.PKV_EUNSUPPORTED),
    (dict(D=96), pkv.PKV_EUNSUPPORTED),
    (dict(Hq=128, Hkv=8), pkv.PKV_EUNSUPPORTED),   # group of 16
    (dict(dtype=7), pkv.PKV_EINVAL),
    (dict(out_dtype=pkv.PKV_F16), pkv.PKV_EINVAL),  # neither f32 nor the input type
    (dict(ps=24), pkv.PKV_EINVAL),                 # not a multiple of the block size
    (dict(ps=-2), pkv.PKV_EINVAL),                 # negative other than the adaptive single pass
    (dict(max_ctx=129), pkv.PKV_EINVAL),           # beyond max_blocks * block_size
    (dict(query=NULL), pkv.PKV_EINVAL),
    (dict(ps=32), pkv.PKV_EINVAL),                 # workspace missing
    (dict(query=(1 << 12) + 2), pkv.PKV_EINVAL),   # misaligned
])
def test_decode_host_validation(kw, status):
    assert _decode(**kw) == status
    assert pkv.last_error()


def test_empty_batch_is_a_no_op():
    assert _decode(B=0) == pkv.PKV_OK
    assert _decode(B=0, ps=512, ws=1 << 12, ws_bytes=1 << 20) == pkv.PKV_OK


def test_workspace_size_formula():
    n = pkv.lib.paged_attention_decode_workspace_bytes(8, 32, 128, 32768, 512)
    parts = 64
    ml = 8 * 32 * parts * 2 * 4
    assert n == ((ml + 255) // 256) * 256 + 8 * 32 * parts * 128 * 4
    assert pkv.lib.paged_attention_decode_workspace_bytes(8, 32, 128, 32768, 0) == 0
    # a context length at the top of the int32 range: the partition count is formed without
    # overflow (ceil((2^31 - 1) / 16) = 2^27 partitions)
    n = pkv.lib.paged_attention_decode_workspace_bytes(1, 1, 64, 2 ** 31 - 1, 16)
    parts = 2 ** 27
    assert n == ((parts * 2 * 4 + 255) // 256) * 256 + parts * 64 * 4


def test_append_and_prefill_host_validation():
    L = pkv.lib
    p = 1 << 12
    assert L.paged_cache_append(p, p, p, p, 0, 0, p, 4, 8, 100, 16, 10, pkv.PKV_BF16, NULL) == pkv.PKV_EUNSUPPORTED
    assert L.paged_cache_append(p, p, p, p, 0, 0, NULL, 4, 8, 128, 16, 10, pkv.PKV_BF16, NULL) == pkv.PKV_EINVAL
    assert L.paged_cache_append(p, p, p, p, 8, 0, p, 4, 8, 128, 16, 10, pkv.PKV_BF16, NULL) == pkv.PKV_EINVAL
    assert L.paged_cache_append(NULL, NULL, NULL, NULL, 0, 0, NULL, 0, 8, 128, 16, 10, pkv.PKV_BF16, NULL) == pkv.PKV_OK
    assert L.paged_attention_prefill_chunk(p, pkv.PKV_F32, p, p, p, p, 0, 16, 32, 8, 96, 16, 64, 0.1, pkv.PKV_F32,
                                           NULL) == pkv.PKV_EUNSUPPORTED
    for bad_scale in (0.0, -0.1, float("inf"), float("nan")):
        assert L.paged_attention_prefill_chunk(p, pkv.PKV_F32, p, p, p, p, 0, 16, 32, 8, 128, 16, 64, bad_scale,
                                               pkv.PKV_BF16, NULL) == pkv.PKV_EINVAL
    assert L.paged_attention_prefill_chunk(p, pkv.PKV_F32, p, p, p, p, 1000, 100, 32, 8, 128, 16, 64, 0.1,
                                           pkv.PKV_BF16, NULL) == pkv.PKV_EINVAL
    assert L.paged_cache_copy_blocks(p, p, NULL, 3, 8, 128, 16, 64, pkv.PKV_BF16, NULL) == pkv.PKV_EINVAL


def test_pool_sanitizer_build(tmp_path):
    """Host pool + builders under AddressSanitizer/UBSan, driven by a seeded operation sequence."""
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    csrc = os.path.join(ROOT, "paged_kv_cache_404_amd", "csrc")
    exe = tmp_path / "pool_fuzz"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", csrc, os.path.join(csrc, "pool.cpp"),
           os.path.join(csrc, "status.cpp"), os.path.join(ROOT, "tests", "native", "pool_fuzz.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0")
    r = subprocess.run([str(exe), "20000"], capture_output=True, text=True, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout


def test_noalloc_decode_rejects_partials_beyond_its_scratch():
    """paged_attention_decode_noalloc refuses, before touching any device, a call whose split-K
    partials exceed the static scratch; the limit is the header's."""
    L = pkv.lib
    assert _lib.PKV_NOALLOC_SCRATCH_BYTES == 16 * 1024 * 1024
    text = open(HEADER).read()
    assert re.search(r"#define PKV_NOALLOC_SCRATCH_BYTES \(16 \* 1024 \* 1024\)", text)
    p = 1 << 12
    need = L.paged_attention_decode_workspace_bytes(64, 32, 128, 65536, 512)
    assert need > _lib.PKV_NOALLOC_SCRATCH_BYTES
    st = L.paged_attention_decode_noalloc(p, pkv.PKV_F32, p, p, p, p, p, 64, 32, 8, 128, 16, 4096, 100000, 65536,
                                          0.1, 512, pkv.PKV_BF16, NULL, NULL)
    assert st == pkv.PKV_EINVAL and "static scratch" in _lib.last_error()


def test_fp8_prefill_and_mixed_host_validation():
    """paged_attention_prefill_chunk_fp8 and paged_attention_mixed_fp8 refuse bad arguments on the
    host (query type, output type, head size, scale, alignment, pool bounds, chunk count) and
    treat empty work as a no-op, all before any launch."""
    L = pkv.lib
    p = 1 << 12
    bf, f32 = pkv.PKV_BF16, pkv.PKV_F32

    def pre(q_dtype=bf, out_dtype=f32, ctx=0, C=16, D=128, scale=0.1, ks=p):
        return L.paged_attention_prefill_chunk_fp8(p, out_dtype, p, p, p, ks, p, p, ctx, C, 32, 8, D, 16, 64, scale,
                                                   q_dtype, NULL)
    assert pre(q_dtype=f32) == pkv.PKV_EUNSUPPORTED
    assert pre(out_dtype=pkv.PKV_F16) == pkv.PKV_EINVAL
    assert pre(D=96) == pkv.PKV_EUNSUPPORTED
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert pre(scale=bad) == pkv.PKV_EINVAL
    assert pre(ctx=1000, C=100) == pkv.PKV_EINVAL       # past the 64-block pool
    assert pre(ks=p + 4) == pkv.PKV_EINVAL              # scales not 16-byte aligned
    assert pre(C=0) == pkv.PKV_OK

    starts = (C.c_int32 * 17)(*([0] * 17))
    lens = (C.c_int32 * 17)(*([16] * 17))

    def mix(q_dtype=bf, out_dtype=f32, n_chunks=1, scale=0.1, ks=p, B=0):
        return L.paged_attention_mixed_fp8(p, p, p, p, B, 4, 64 if B else 0, NULL, 0, NULL, 0, p, p, p, 8, starts,
                                           lens, n_chunks, out_dtype, p, p, ks, p, 32, 8, 128, 16, 64, scale, q_dtype,
                                           NULL)
    assert mix(q_dtype=f32) == pkv.PKV_EUNSUPPORTED
    assert mix(out_dtype=pkv.PKV_F16) == pkv.PKV_EINVAL
    assert mix(n_chunks=17) == pkv.PKV_EUNSUPPORTED
    assert mix(scale=0.0) == pkv.PKV_EINVAL
    assert mix(ks=NULL) == pkv.PKV_EINVAL
    assert mix(ks=p + 4) == pkv.PKV_EINVAL
    assert mix(B=2, n_chunks=0, out_dtype=pkv.PKV_F16) == pkv.PKV_EINVAL
    assert mix(n_chunks=0) == pkv.PKV_OK                # nothing to do


def test_mixed_host_validation():
    """paged_attention_mixed: fp32 caches are accepted but not grouped; an unknown dtype and a
    group size other than 1 or the 8-column size are refused; nothing to do is a no-op."""
    L = pkv.lib
    p = 1 << 12
    starts = (C.c_int32 * 1)(0)
    lens = (C.c_int32 * 1)(16)

    def mix(dtype=pkv.PKV_BF16, out_dtype=pkv.PKV_F32, group=1, n_chunks=1, B=0):
        return L.paged_attention_mixed(p, p, p, p, B, 4, 64 if B else 0, NULL, 0, group, NULL, 0, p, p, p, 8, starts,
                                       lens, n_chunks, out_dtype, p, p, 32, 8, 128, 16, 64, 0.1, dtype, NULL)
    assert mix(dtype=7) == pkv.PKV_EUNSUPPORTED
    assert mix(dtype=pkv.PKV_F32, group=2, B=2) == pkv.PKV_EUNSUPPORTED
    assert mix(group=3, B=2) == pkv.PKV_EUNSUPPORTED
    assert mix(dtype=pkv.PKV_F32, n_chunks=0) == pkv.PKV_OK
    assert mix(n_chunks=0) == pkv.PKV_OK
