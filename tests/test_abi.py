"""C ABI: the library loads, exports every declared symbol, and rejects bad
arguments on the host before any HIP call (runs without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def _lib():
    import attention_fa_fwd_03_amd as fa
    return fa


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(fa_[a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["fa_fwd_dense", "fa_fwd_varlen", "fa_fwd_paged", "fa_fwd_paged_vec", "fa_fwd_paged_ex",
              "fa_fwd_paged_workspace_size",
              "fa_last_error", "fa_abi_version"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    fa = _lib()
    raw = ctypes.CDLL(fa.library_path)
    for n in declared_functions():
        assert hasattr(raw, n), n


def test_header_compiles_as_c():
    import subprocess
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "t.c")
        with open(src, "w") as f:
            f.write('#include "fa.h"\nint main(void){ fa_mods m = {0}; (void)m; return 0; }\n')
        r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), "-c", src,
                            "-o", os.path.join(d, "t.o")], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


FAKE = 1 << 20   # host validation never dereferences pointers


def _dense(**kw):
    fa = _lib()
    a = dict(q=FAKE, k=FAKE * 2, v=FAKE * 3, o=FAKE * 4, lse=FAKE * 5, B=1, Sq=4, Skv=4, Hq=2, Hkv=2,
             dqk=64, dv=64, mods=None)
    a.update(kw)
    rc = fa.lib.fa_fwd_dense(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Sq"], a["Skv"], a["Hq"], a["Hkv"],
                             a["dqk"], a["dv"], a["mods"], None)
    return rc, fa.fa_last_error()


@pytest.mark.parametrize("kw,code,frag", [
    (dict(Hq=3, Hkv=2), -1, "multiple"),
    (dict(Hkv=0), -1, "positive"),
    (dict(B=-1), -1, "B must"),
    (dict(dqk=96, dv=96), -2, "not built"),
    (dict(dqk=192, dv=128), -2, "not built"),
    (dict(q=0), -1, "non-NULL"),
    (dict(lse=0), -1, "non-NULL"),
    (dict(Sq=1 << 31), -3, "2^31"),
])
def test_dense_rejects(kw, code, frag):
    rc, msg = _dense(**kw)
    assert rc == code and frag in msg, (rc, msg)


@pytest.mark.parametrize("kw", [dict(q=FAKE + 8), dict(v=FAKE * 3 + 4), dict(o=FAKE * 4 + 2), dict(lse=FAKE * 5 + 2)])
def test_dense_rejects_misaligned_pointers(kw):
    rc, msg = _dense(**kw)
    assert rc == -1 and "aligned" in msg, (rc, msg)


def test_dense_rejects_lse_overlapping_o():
    rc, msg = _dense(o=FAKE * 4, lse=FAKE * 4 + 8)
    assert rc == -1 and "overlap" in msg


def test_empty_batch_is_a_no_op():
    rc, _ = _dense(B=0, q=0, k=0, v=0, o=0, lse=0)
    assert rc == 0
    rc, _ = _dense(Sq=0, q=0, k=0, v=0, o=0, lse=0)
    assert rc == 0


def test_mods_validation():
    fa = _lib()
    m = fa.Mods(softcap=-1.0).to_c()
    rc, msg = _dense(mods=ctypes.byref(m))
    assert rc == -1 and "softcap" in msg
    m = fa.Mods().to_c()
    m.flags = fa.FA_BLOCK_MASK
    m.block_mask = FAKE * 9
    m.mask_block_q, m.mask_block_k, m.mask_nqb, m.mask_nkb = 64, 64, 1, 1
    rc, msg = _dense(mods=ctypes.byref(m))
    assert rc == -2 and "multiples" in msg
    m.mask_block_q, m.mask_block_k, m.mask_nqb, m.mask_nkb = 128, 64, 0, 1
    rc, msg = _dense(mods=ctypes.byref(m))
    assert rc == -1 and "cover" in msg
    m = fa.Mods().to_c()
    m.flags = 1 << 7
    rc, msg = _dense(mods=ctypes.byref(m))
    assert rc == -1 and "unknown" in msg


def _paged(vec=False, opts=None, **kw):
    fa = _lib()
    a = dict(q=FAKE, kc=FAKE * 2, vc=FAKE * 3, o=FAKE * 4, lse=FAKE * 5, cu=FAKE * 6, sk=FAKE * 7, bt=FAKE * 8,
             B=2, Tq=2, msq=1, msk=100, P=10, ps=64, mp=2, Hq=16, Hkv=2, dqk=192, dv=128, kv=1,
             kd=FAKE * 9, vd=FAKE * 10, ws=FAKE * 64, wsb=1 << 30, mods=None)
    a.update(kw)
    fn = fa.lib.fa_fwd_paged_vec if vec else fa.lib.fa_fwd_paged
    if opts is not None:
        fn = lambda *x: fa.lib.fa_fwd_paged_ex(*x[:-2], ctypes.byref(opts), *x[-2:])
    rc = fn(a["q"], a["kc"], a["vc"], a["o"], a["lse"], a["cu"], a["sk"], a["bt"], a["B"], a["Tq"],
            a["msq"], a["msk"], a["P"], a["ps"], a["mp"], a["Hq"], a["Hkv"], a["dqk"], a["dv"],
            a["kv"], a["kd"], a["vd"], a["ws"], a["wsb"], a["mods"], None)
    return rc, fa.fa_last_error()


@pytest.mark.parametrize("kw,code,frag", [
    (dict(ps=48), -2, "power of two"),
    (dict(ps=2048), -2, "power of two"),
    (dict(mp=1), -1, "max_pages_per_seq"),
    (dict(kd=0), -1, "descale"),
    (dict(ws=0), -4, "workspace"),
    (dict(wsb=16), -4, "workspace"),
    (dict(kv=7), -1, "kv_dtype"),
    (dict(P=1 << 31), -3, "2^31"),
    (dict(Tq=1 << 31, msq=1), -3, "2^31"),
    (dict(dqk=256, dv=256, msq=100, Tq=200), -2, "not built"),
    (dict(bt=0), -1, "non-NULL"),
])
def test_paged_rejects(kw, code, frag):
    rc, msg = _paged(**kw)
    assert rc == code and frag in msg, (rc, msg)


@pytest.mark.parametrize("kw", [dict(kc=FAKE * 2 + 8), dict(bt=FAKE * 8 + 2), dict(ws=FAKE * 64 + 4)])
def test_paged_rejects_misaligned_pointers(kw):
    rc, msg = _paged(**kw)
    assert rc == -1 and "aligned" in msg, (rc, msg)


@pytest.mark.parametrize("kw,code,frag", [
    (dict(kv=0), -2, "FP8"),
    (dict(ps=8, mp=16), -2, "page_size >= 16"),
    (dict(ps=1, mp=128), -2, "page_size >= 16"),
    (dict(ps=48), -2, "power of two"),
    (dict(mp=1), -1, "max_pages_per_seq"),
    (dict(ws=0), -4, "workspace"),
    (dict(dqk=256, dv=256, msq=100, Tq=200), -2, "not built"),
])
def test_paged_vec_rejects(kw, code, frag):
    """The vectorised format holds FP8 whole 16-key blocks; every other check
    is the head-major entry point's."""
    rc, msg = _paged(vec=True, **kw)
    assert rc == code and frag in msg, (rc, msg)


def _opts(q_dtype=1, q_descale=FAKE * 11, layout=0):
    from attention_fa_fwd_03_amd.binding import _FaPagedOpts
    return _FaPagedOpts(q_dtype, q_descale, layout)


@pytest.mark.parametrize("opt_kw,kw,code,frag", [
    (dict(q_descale=0), dict(), -1, "q_descale"),
    (dict(), dict(kv=0), -2, "FP8 E4M3 cache"),
    (dict(q_dtype=5), dict(), -1, "q_dtype"),
    (dict(layout=2), dict(), -1, "page_layout"),
    (dict(layout=1), dict(ps=8, mp=16), -2, "page_size >= 16"),
    (dict(q_dtype=0, layout=1), dict(kv=0), -2, "FP8"),
])
def test_paged_ex_rejects(opt_kw, kw, code, frag):
    rc, msg = _paged(opts=_opts(**opt_kw), **kw)
    assert rc == code and frag in msg, (rc, msg)


@pytest.mark.parametrize("target", ["q", "o", "lse", "cu", "sk", "bt", "kc", "vc", "kd", "vd"])
def test_paged_decode_workspace_must_not_overlap(target):
    """The decode path's plan kernel writes the workspace while the call
    reads the metadata, the caches and the descales and writes O and LSE."""
    base = dict(q=FAKE, kc=FAKE * 2, vc=FAKE * 3, o=FAKE * 4, lse=FAKE * 5, cu=FAKE * 6, sk=FAKE * 7, bt=FAKE * 8,
                kd=FAKE * 9, vd=FAKE * 10)
    rc, msg = _paged(ws=base[target])
    assert rc == -1 and "overlap" in msg, (target, rc, msg)


@pytest.mark.parametrize("mkw,code,frag", [
    (dict(softcap=-1.0), -1, "softcap"),
    (dict(alibi_slope=float("inf")), -1, "alibi_slope"),
    (dict(block_mask="bq64"), -2, "multiples"),
    (dict(block_mask="short"), -1, "does not cover"),
])
def test_paged_checks_mod_parameters(mkw, code, frag):
    """FP8 paged calls take every score mod; their parameters are checked as
    for the dense entry point, before any device work (every case here is
    rejected, so no kernel is launched on the placeholder pointers)."""
    fa = _lib()
    bm = mkw.pop("block_mask", None)
    m = fa.Mods(**mkw).to_c()
    if bm is not None:
        # the struct directly: the Python wrapper wants a device tensor
        m.flags |= fa.FA_BLOCK_MASK
        m.block_mask = FAKE * 12
        m.mask_block_q, m.mask_block_k = (64, 64) if bm == "bq64" else (128, 64)
        m.mask_nqb, m.mask_nkb = 1, 1   # "short": 1 key block cannot cover 100 keys
    rc, msg = _paged(mods=ctypes.byref(m))
    assert rc == code and frag in msg, (rc, msg)


def test_workspace_size_query():
    fa = _lib()
    # decode shape: rows = 1 query x 8 q-heads per kv-head <= 32
    n = fa.fa_fwd_paged_workspace_size(64, 64, 1, 32768, 64, 8, 192, 128, 64)
    assert n > 64 * 64 * 129 * 4
    # prefill shape needs none
    assert fa.fa_fwd_paged_workspace_size(4, 8192, 2048, 2048, 16, 16, 192, 128, 64) == 0
    # bf16 caches never take the split path
    assert fa.fa_fwd_paged_workspace_size(64, 64, 1, 32768, 64, 8, 192, 128, 64, fa.FA_BF16) == 0


def _kvw(**kw):
    fa = _lib()
    a = dict(k=FAKE, v=FAKE * 2, sm=FAKE * 3, T=10, Hkv=2, dqk=192, dv=128, kc=FAKE * 4, vc=FAKE * 40,
             P=4, ps=64, layout=0, kd=FAKE * 80, vd=FAKE * 81, mode=1, ws=FAKE * 90, wsb=1 << 20)
    a.update(kw)
    rc = fa.lib.fa_kv_cache_write_fp8(a["k"], a["v"], a["sm"], a["T"], a["Hkv"], a["dqk"], a["dv"], a["kc"], a["vc"],
                                      a["P"], a["ps"], a["layout"], a["kd"], a["vd"], a["mode"], a["ws"], a["wsb"],
                                      None)
    return rc, fa.fa_last_error()


@pytest.mark.parametrize("kw,code,frag", [
    (dict(dqk=200), -2, "multiples of 16"),
    (dict(layout=3), -1, "page_layout"),
    (dict(mode=2), -1, "scale_mode"),
    (dict(layout=1, ps=8), -2, "[16, 1024]"),
    (dict(ps=48), -2, "power of two"),
    (dict(ws=0), -4, "workspace"),
    (dict(wsb=4), -4, "workspace"),
    (dict(sm=0), -1, "non-NULL"),
    (dict(vd=FAKE * 80), -1, "differ"),
    (dict(T=-1), -1, ">= 0"),
])
def test_kv_cache_write_rejects(kw, code, frag):
    rc, msg = _kvw(**kw)
    assert rc == code and frag in msg, (rc, msg)


@pytest.mark.parametrize("kw", [dict(k=FAKE + 8), dict(sm=FAKE * 3 + 4), dict(vc=FAKE * 40 + 1)])
def test_kv_cache_write_rejects_misaligned_pointers(kw):
    rc, msg = _kvw(**kw)
    assert rc == -1 and "aligned" in msg, (rc, msg)


def test_kv_cache_write_empty_and_workspace_query():
    fa = _lib()
    assert _kvw(T=0, k=0, v=0, sm=0, ws=0)[0] == 0
    assert fa.fa_kv_cache_write_fp8_workspace_size(0, 8, 192, 128) == 0
    n = fa.fa_kv_cache_write_fp8_workspace_size(1000, 8, 192, 128)
    assert 0 < n < 1 << 16 and n % 4 == 0


def _bwd(**kw):
    fa = _lib()
    a = dict(B=1, Sq=16, Skv=16, Hq=2, Hkv=2, dqk=64, dv=64, mods=None, ws=FAKE * 30, wsb=1 << 20)
    a.update(kw)
    ptrs = [FAKE * (i + 1) for i in range(9)]
    rc = fa.lib.fa_bwd_dense(*ptrs, a["B"], a["Sq"], a["Skv"], a["Hq"], a["Hkv"], a["dqk"], a["dv"], a["mods"],
                             a["ws"], a["wsb"], None)
    return rc, fa.fa_last_error()


@pytest.mark.parametrize("kw,code,frag", [
    (dict(dqk=192, dv=128), -2, "not built"),
    (dict(dqk=128, dv=64), -2, "not built"),
    (dict(ws=0), -4, "workspace"),
    (dict(wsb=8), -4, "workspace"),
    (dict(Hq=3, Hkv=2), -1, "multiple"),
    (dict(Sq=-1), -1, ">= 0"),
    (dict(Hq=131072, Hkv=131072, dqk=128, dv=128), -3, "2^24"),
])
def test_bwd_rejects(kw, code, frag):
    rc, msg = _bwd(**kw)
    assert rc == code and frag in msg, (rc, msg)


def test_bwd_rejects_misaligned_pointers():
    fa = _lib()
    ptrs = [FAKE * (i + 1) for i in range(9)]
    ptrs[6] += 8    # dq
    rc = fa.lib.fa_bwd_dense(*ptrs, 1, 16, 16, 2, 2, 64, 64, None, FAKE * 30, 1 << 20, None)
    assert rc == -1 and "aligned" in fa.fa_last_error()


def test_bwd_rejects_score_mods_and_overlap():
    fa = _lib()
    m = fa.Mods(softcap=20.0).to_c()
    rc, msg = _bwd(mods=ctypes.byref(m))
    assert rc == -2 and "FA_CAUSAL" in msg
    ptrs = [FAKE * (i + 1) for i in range(9)]
    ptrs[6] = ptrs[0]                      # dq aliases q
    rc = fa.lib.fa_bwd_dense(*ptrs, 1, 16, 16, 2, 2, 64, 64, None, FAKE * 30, 1 << 20, None)
    assert rc == -1 and "overlap" in fa.fa_last_error()
    assert fa.fa_bwd_workspace_size(0, 4) == 0 and fa.fa_bwd_workspace_size(10, 4) == 160


def _noalloc(**kw):
    fa = _lib()
    a = dict(q=FAKE, kc=FAKE * 2, vc=FAKE * 3, o=FAKE * 4, lse=FAKE * 5, cu=FAKE * 6, sk=FAKE * 7, bt=FAKE * 8,
             B=2, Tq=2, msq=1, msk=100, P=10, ps=64, mp=2, Hq=16, Hkv=2, dqk=192, dv=128, kv=1,
             kd=FAKE * 9, vd=FAKE * 10, mods=None)
    a.update(kw)
    rc = fa.lib.fa_fwd_paged_noalloc(a["q"], a["kc"], a["vc"], a["o"], a["lse"], a["cu"], a["sk"], a["bt"], a["B"],
                                     a["Tq"], a["msq"], a["msk"], a["P"], a["ps"], a["mp"], a["Hq"], a["Hkv"],
                                     a["dqk"], a["dv"], a["kv"], a["kd"], a["vd"], a["mods"], None)
    return rc, fa.fa_last_error()


@pytest.mark.parametrize("kw,code,frag", [
    (dict(ps=48), -2, "power of two"),
    (dict(kd=0), -1, "descale"),
    (dict(bt=0), -1, "non-NULL"),
    # a decode call whose scratch need exceeds the static 64 MiB array
    (dict(B=4096, Tq=4096, msk=1 << 20, mp=(1 << 20) // 64, Hq=64, Hkv=8,
          **{n: (i + 1) << 30 for i, n in enumerate(["q", "kc", "vc", "o", "lse", "cu", "sk", "bt", "kd", "vd"])}),
     -3, "scratch"),
])
def test_paged_noalloc_rejects(kw, code, frag):
    """The no-allocation entry point validates like fa_fwd_paged (before any
    HIP call) and refuses decode calls whose scratch exceeds its array."""
    rc, msg = _noalloc(**kw)
    assert rc == code and frag in msg, (rc, msg)


def test_paged_noalloc_limit_matches_the_workspace_query():
    fa = _lib()
    need = fa.fa_fwd_paged_workspace_size(4096, 4096, 1, 1 << 20, 64, 8, 192, 128, 64)
    assert need > 64 << 20
    assert fa.fa_fwd_paged_workspace_size(64, 64, 1, 32768, 64, 8, 192, 128, 64) <= 64 << 20
