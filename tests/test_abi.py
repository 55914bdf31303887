"""C-ABI checks that need no GPU: the library loads, exports every function
include/sikv.h declares, its descriptor layout matches, and host-side argument
validation rejects bad calls before anything is launched.

Every call below is invalid by construction (it fails a host check), so no
kernel is ever launched and the fake device addresses are never dereferenced.
"""

import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sikv.h")

sk = pytest.importorskip("bit_self_indexed_amd")
from bit_self_indexed_amd import _abi  # noqa: E402

lib = sk.lib
OK, INVALID, UNSUPPORTED, WORKSPACE, HIP = 0, -1, -2, -3, -4
FAKE = 0x10000000  # 256-byte aligned fake device address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^[a-z_0-9 ]+\**\s*\**(sikv_\w+)\(", text, re.M)))


def test_header_functions_are_exported_and_declared():
    names = declared_functions()
    assert "sikv_encode" in names and "sikv_decode_step" in names
    assert set(names) == set(_abi.SIGNATURES)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_desc_layout():
    assert lib.sikv_abi_version() == _abi.ABI_VERSION
    assert lib.sikv_desc_size() == C.sizeof(_abi.CacheDesc) == 152
    offs = {f[0]: getattr(_abi.CacheDesc, f[0]).offset for f in _abi.CacheDesc._fields_}
    assert offs["codes"] == 24 and offs["v"] == 56 and offs["v_stride_t"] == 80
    assert offs["codebook"] == 88 and offs["vrec"] == 96 and offs["v_sink"] == 104
    assert offs["seq_lens"] == 112 and offs["page_table"] == 120 and offs["n_pages"] == 136
    assert offs["flags"] == 140 and offs["timer"] == 144


def test_status_strings():
    for code in (OK, INVALID, UNSUPPORTED, WORKSPACE, HIP):
        s = lib.sikv_status_str(code).decode()
        assert s and s != "unknown status"
    assert lib.sikv_status_str(-99).decode() == "unknown status"


def desc(**kw):
    d = _abi.CacheDesc()
    d.batch, d.n_kv_heads, d.head_dim, d.capacity, d.n_tokens, d.n_sink = 2, 2, 128, 1000, 900, 64
    d.codes, d.alpha, d.mu, d.k_sink = FAKE, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000
    d.v, d.v_stride_b, d.v_stride_h, d.v_stride_t = FAKE + 0x400000, 2 * 1000 * 128, 1000 * 128, 128
    d.codebook = d.vrec = d.v_sink = d.seq_lens = d.page_table = None
    d.page_size = d.pages_per_seq = d.n_pages = d.flags = 0
    d.timer = None
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def score(d, q=FAKE, hq=4, k=16, idx=FAKE, ws=None, wsn=0):
    return lib.sikv_score_topk(C.byref(d), q, hq, k, idx, None, ws, wsn, None)


def test_workspace_sizes():
    d = desc()
    assert lib.sikv_workspace_bytes(0, C.byref(d), 1, 1) > 0
    s1 = lib.sikv_workspace_bytes(1, C.byref(d), 4, 16)
    s2 = lib.sikv_workspace_bytes(2, C.byref(d), 4, 16)
    s3 = lib.sikv_workspace_bytes(3, C.byref(d), 4, 16)
    assert s1 > 0 and s2 > 0 and s3 >= s1 + s2
    assert lib.sikv_workspace_bytes(1, C.byref(d), 3, 16) == 0          # Hq % Hkv
    assert lib.sikv_workspace_bytes(1, C.byref(d), 4, 837) == 0         # k > N - 64
    assert lib.sikv_workspace_bytes(9, C.byref(d), 4, 16) == 0          # bad op
    assert lib.sikv_workspace_bytes(1, None, 4, 16) == 0
    big = desc(capacity=600000, n_tokens=524288, batch=1, n_kv_heads=8)
    assert lib.sikv_workspace_bytes(3, C.byref(big), 40, 4096) > 0
    # prefill with a codebook needs room for the per-block cluster statistics
    cbd = desc(codebook=FAKE + 0x500000)
    assert (lib.sikv_workspace_bytes(0, C.byref(cbd), 1, 1)
            >= lib.sikv_workspace_bytes(0, C.byref(d), 1, 1) + 2 * 2 * 1 * 2560 * 8)
    assert lib.sikv_dense_workspace_bytes(4, 8, 32, 131072) > 0
    assert lib.sikv_dense_workspace_bytes(4, 8, 30, 131072) == 0


@pytest.mark.parametrize("field,value,expect", [
    ("head_dim", 64, UNSUPPORTED),
    ("n_sink", 32, UNSUPPORTED),
    ("codebook", FAKE + 4, INVALID),                                # misaligned
    ("n_tokens", 64, INVALID),
    ("n_tokens", 1001, INVALID),
    ("batch", 0, INVALID),
    ("codes", None, INVALID),
    ("codes", FAKE + 8, INVALID),
    ("mu", FAKE + 4, INVALID),
    ("alpha", FAKE + 2, INVALID),
    ("vrec", FAKE + 0x600000, INVALID),                             # v_sink missing
    ("v_sink", FAKE + 0x600000, INVALID),
    ("seq_lens", FAKE + 2, INVALID),                                # misaligned
    ("flags", 2, INVALID),                                          # unknown flag bit
    ("flags", -1, INVALID),
])
def test_descriptor_validation(field, value, expect):
    d = desc(**{field: value})
    assert score(d) == expect


def test_query_validation():
    d = desc()
    assert score(d, q=None) == INVALID
    assert score(d, q=FAKE + 2) == INVALID
    assert score(d, hq=3) == INVALID           # not a multiple of Hkv
    assert score(d, hq=18) == UNSUPPORTED      # G = 9
    assert score(d, k=0) == INVALID
    assert score(d, k=837) == INVALID          # N - 64 = 836
    assert score(d, idx=None) == INVALID
    assert score(d) == WORKSPACE               # no workspace
    need = lib.sikv_workspace_bytes(1, C.byref(d), 4, 16)
    assert score(d, ws=FAKE, wsn=need - 1) == WORKSPACE
    assert score(d, ws=FAKE + 64, wsn=need) == WORKSPACE   # misaligned


def test_attention_and_decode_validation():
    d = desc()
    nd = desc(v=None)
    sd = desc(v_stride_t=100)
    f = C.c_float
    for dd in (nd, sd):
        assert lib.sikv_sparse_attn(C.byref(dd), FAKE, 4, FAKE, 16, f(0.088), FAKE, FAKE, 1 << 30,
                                    None) == INVALID
        assert lib.sikv_decode_step(C.byref(dd), FAKE, 4, 16, f(0.088), None, FAKE, FAKE, 1 << 30,
                                    None) == INVALID
    assert lib.sikv_sparse_attn(C.byref(d), FAKE, 4, FAKE, 16, f(float("nan")), FAKE, FAKE,
                                1 << 30, None) == INVALID
    assert lib.sikv_sparse_attn(C.byref(d), FAKE, 4, None, 16, f(0.088), FAKE, FAKE, 1 << 30,
                                None) == INVALID
    assert lib.sikv_decode_step(C.byref(d), FAKE, 4, 16, f(0.088), None, None, FAKE, 1 << 30,
                                None) == INVALID
    need = lib.sikv_workspace_bytes(3, C.byref(d), 4, 16)
    assert lib.sikv_decode_step(C.byref(d), FAKE, 4, 16, f(0.088), None, FAKE, FAKE, need - 256,
                                None) == WORKSPACE


def test_append_decode_validation():
    d = desc()
    f = C.c_float
    need = lib.sikv_workspace_bytes(3, C.byref(d), 4, 16)
    # missing or misaligned new key row, bad strides: rejected before any launch
    assert lib.sikv_append_decode_step(C.byref(d), None, 1024, 128, None, 0, 0, FAKE, 4, 16, f(0.088), None,
                                       FAKE, FAKE, need, None) == INVALID
    assert lib.sikv_append_decode_step(C.byref(d), FAKE + 2, 1024, 128, None, 0, 0, FAKE, 4, 16, f(0.088),
                                       None, FAKE, FAKE, need, None) == INVALID
    assert lib.sikv_append_decode_step(C.byref(d), FAKE, 1024, 100, None, 0, 0, FAKE, 4, 16, f(0.088), None,
                                       FAKE, FAKE, need, None) == INVALID
    assert lib.sikv_append_decode_step(C.byref(d), FAKE, 1024, 128, None, 0, 0, FAKE, 4, 16, f(0.088), None,
                                       FAKE, FAKE, need - 256, None) == WORKSPACE
    nd = desc(v=None)
    assert lib.sikv_append_decode_step(C.byref(nd), FAKE, 1024, 128, None, 0, 0, FAKE, 4, 16, f(0.088), None,
                                       FAKE, FAKE, need, None) == INVALID


def test_quantised_value_validation():
    f = C.c_float
    qd = desc(v=None, vrec=FAKE + 0x600000, v_sink=FAKE + 0x800000)
    d = desc()
    need = lib.sikv_workspace_bytes(3, C.byref(qd), 4, 16)
    assert need > 0
    # v_new only with quantised values; aligned, strides multiples of 8
    assert lib.sikv_append_decode_step(C.byref(d), FAKE, 1024, 128, FAKE, 1024, 128, FAKE, 4, 16,
                                       f(0.088), None, FAKE, FAKE, need, None) == INVALID
    assert lib.sikv_append_decode_step(C.byref(qd), FAKE, 1024, 128, FAKE + 2, 1024, 128, FAKE,
                                       4, 16, f(0.088), None, FAKE, FAKE, need, None) == INVALID
    assert lib.sikv_append_decode_step(C.byref(qd), FAKE, 1024, 128, FAKE, 1024, 12, FAKE, 4, 16,
                                       f(0.088), None, FAKE, FAKE, need, None) == INVALID
    assert lib.sikv_append_decode_step(C.byref(qd), FAKE, 1024, 128, FAKE, 1024, 128, FAKE, 4, 16,
                                       f(0.088), None, FAKE, FAKE, need - 256, None) == WORKSPACE
    ev = lib.sikv_encode_v
    assert ev(C.byref(d), FAKE, 0, 0, 128, 0, 10, None) == INVALID          # no vq
    assert ev(C.byref(qd), None, 0, 0, 128, 0, 10, None) == INVALID
    assert ev(C.byref(qd), FAKE + 2, 0, 0, 128, 0, 10, None) == INVALID
    assert ev(C.byref(qd), FAKE, 0, 0, 100, 0, 10, None) == INVALID         # stride
    assert ev(C.byref(qd), FAKE, 0, 0, 128, 10, 10, None) == INVALID        # empty
    assert ev(C.byref(qd), FAKE, 0, 0, 128, -1, 10, None) == INVALID
    assert ev(C.byref(qd), FAKE, 0, 0, 128, 0, 1001, None) == INVALID       # > capacity
    assert lib.sikv_encode_v(None, FAKE, 0, 0, 128, 0, 10, None) == INVALID
    misal = desc(v=None, vrec=FAKE + 0x600010, v_sink=FAKE + 0x800000)         # not 64-aligned
    assert score(misal) == INVALID


def test_static_scratch_entry_point_validation():
    """sikv_append_decode_step_static checks everything before it touches the
    GPU: bad arguments and a workspace need above the static scratch size are
    rejected with nothing launched (the size comes from the header)."""
    f = C.c_float
    st = lib.sikv_append_decode_step_static
    d = desc()
    assert st(C.byref(d), None, 1024, 128, None, 0, 0, FAKE, 4, 16, f(0.088), None, FAKE,
              None) == INVALID
    assert st(C.byref(d), FAKE, 1024, 100, None, 0, 0, FAKE, 4, 16, f(0.088), None, FAKE,
              None) == INVALID
    assert st(C.byref(d), FAKE, 1024, 128, None, 0, 0, FAKE, 4, 16, f(0.088), None, None,
              None) == INVALID
    assert st(None, FAKE, 1024, 128, None, 0, 0, FAKE, 4, 16, f(0.088), None, FAKE,
              None) == INVALID
    limit = int(re.search(r"#define SIKV_STATIC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)",
                          open(HEADER).read()).expand(r"\1 \2").split()[0]) << 20
    # 4 x 8 KV heads at 128K tokens fit; 8 x 8 heads at 512K do not
    fits = desc(batch=4, n_kv_heads=8, capacity=131072, n_tokens=131072, v_stride_b=8 * 131072 * 128,
                v_stride_h=131072 * 128)
    big = desc(batch=8, n_kv_heads=8, capacity=524288, n_tokens=524288, v_stride_b=8 * 524288 * 128,
               v_stride_h=524288 * 128)
    assert 0 < lib.sikv_workspace_bytes(3, C.byref(fits), 32, 9830) <= limit
    assert lib.sikv_workspace_bytes(3, C.byref(big), 32, 4096) > limit
    assert st(C.byref(big), FAKE, 1024, 128, None, 0, 0, FAKE, 32, 4096, f(0.088), None, FAKE,
              None) == WORKSPACE


def test_encode_validation():
    d = desc()
    e = lib.sikv_encode
    assert e(C.byref(d), None, 0, 0, 128, 0, 900, 1, FAKE, 1 << 30, None) == INVALID
    assert e(C.byref(d), FAKE + 2, 0, 0, 128, 0, 900, 1, FAKE, 1 << 30, None) == INVALID
    assert e(C.byref(d), FAKE, 0, 0, 100, 0, 900, 1, FAKE, 1 << 30, None) == INVALID  # stride
    assert e(C.byref(d), FAKE, 0, 0, 128, 1, 900, 1, FAKE, 1 << 30, None) == INVALID  # t_begin
    assert e(C.byref(d), FAKE, 0, 0, 128, 0, 899, 1, FAKE, 1 << 30, None) == INVALID  # t_end != N
    assert e(C.byref(d), FAKE, 0, 0, 128, 0, 900, 2, FAKE, 1 << 30, None) == INVALID
    assert e(C.byref(d), FAKE, 0, 0, 128, 0, 900, 1, None, 0, None) == WORKSPACE
    assert e(C.byref(d), FAKE, 0, 0, 128, 900, 1001, 0, None, 0, None) == INVALID     # > capacity
    assert e(C.byref(d), FAKE, 0, 0, 128, 900, 900, 0, None, 0, None) == INVALID      # empty


def test_dense_and_copy_validation():
    f = C.c_float
    assert lib.sikv_dense_attn(1, 2, 3, 100, FAKE, FAKE, 0, 0, 128, FAKE, 0, 0, 128, f(0.1), FAKE,
                               FAKE, 1 << 30, None, None) == INVALID
    assert lib.sikv_dense_attn(1, 1, 9, 100, FAKE, FAKE, 0, 0, 128, FAKE, 0, 0, 128, f(0.1), FAKE,
                               FAKE, 1 << 30, None, None) == UNSUPPORTED
    assert lib.sikv_dense_attn(1, 1, 4, 100, FAKE, FAKE, 0, 0, 128, FAKE, 0, 0, 128, f(0.1), FAKE,
                               None, 0, None, None) == WORKSPACE
    assert lib.sikv_stream_copy(FAKE, FAKE, 17, None, None) == INVALID
    assert lib.sikv_stream_copy(None, FAKE, 16, None, None) == INVALID


def test_timer_without_launches():
    """A caller-owned timer: created, read (nothing launched), reset, destroyed;
    two timers are independent objects."""
    assert lib.sikv_timer_count() >= 10
    names = [lib.sikv_timer_name(i).decode() for i in range(lib.sikv_timer_count())]
    assert "score" in names and "attn" in names
    assert lib.sikv_timer_name(99).decode() == "unknown"
    t1, t2 = C.c_void_p(), C.c_void_p()
    assert lib.sikv_timer_create(C.byref(t1)) == OK and t1.value
    assert lib.sikv_timer_create(C.byref(t2)) == OK and t2.value and t2.value != t1.value
    n, ms = C.c_int64(), C.c_double()
    assert lib.sikv_timer_read(t1, 0, C.byref(n), C.byref(ms)) == OK and n.value == 0
    assert lib.sikv_timer_read(t1, 99, C.byref(n), C.byref(ms)) == INVALID
    assert lib.sikv_timer_read(None, 0, C.byref(n), C.byref(ms)) == INVALID
    assert lib.sikv_timer_reset(t1) == OK and lib.sikv_timer_reset(None) == INVALID
    assert lib.sikv_timer_create(None) == INVALID
    assert lib.sikv_timer_destroy(t1) == OK and lib.sikv_timer_destroy(t2) == OK
    assert lib.sikv_timer_destroy(None) == OK


# Writable symbols that the toolchain and the HIP runtime put into every
# shared library: ELF/C++ runtime bookkeeping, HIP's code-object registration
# (fat binary wrappers, module handles, compilation-unit ids) and one host-side
# handle per kernel, named after the kernel.
_TOOLCHAIN_SYMBOLS = re.compile(
    r"^(_DYNAMIC|_GLOBAL_OFFSET_TABLE_|__dso_handle|__init|__fini|__do_(init|fini)\.\w+"
    r"|DW\.ref\.\w+|__hip_(fatbin_wrapper|gpubin_handle_\w+|cuid_\w+))$"
    r"|::\w+_kernel(<[^>]*>)?\(")
# The one exception, by design: the allocation-free entry point's static device
# scratch (its host stand-in) and the per-device address of it, set once.
_STATIC_SCRATCH = re.compile(r"^\(anonymous namespace\)::(scratch|g_scratch)$")


def test_library_has_no_mutable_globals():
    """The C ABI keeps no state between calls: apart from what the toolchain and
    HIP put into every library and the allocation-free entry point's static
    scratch, its writable data segments hold nothing (the timer and the
    exact-selection switch are caller-owned)."""
    import subprocess
    nm = subprocess.run(["nm", "-C", "--defined-only", sk.LIB_PATH], capture_output=True,
                        text=True)
    if nm.returncode != 0:
        pytest.skip("nm unavailable")
    writable = [l.split(" ", 2)[2] for l in nm.stdout.splitlines()
                if re.match(r"^[0-9a-f]+ [bBdD] ", l)]
    assert writable, "no writable symbols listed at all: the nm output format changed"
    own = [n for n in writable
           if not _TOOLCHAIN_SYMBOLS.search(n) and not _STATIC_SCRATCH.search(n)]
    assert not own, own


def test_paged_descriptor_validation():
    """Page size a power of two >= 256, capacity = pages_per_seq * page_size,
    a row count that fits int32, the bf16 V pool dense in the page layout."""
    ok = dict(page_table=FAKE + 0x900000, page_size=256, pages_per_seq=4, n_pages=16,
              capacity=1024, n_tokens=900, v_stride_b=2 * 256 * 128, v_stride_h=256 * 128,
              v_stride_t=128)
    assert score(desc(**ok)) == WORKSPACE                    # valid: fails only for workspace
    f = C.c_float
    attn = lambda d: lib.sikv_sparse_attn(C.byref(d), FAKE, 4, FAKE, 16, f(0.088), FAKE, None, 0,
                                          None)
    assert attn(desc(**ok)) == WORKSPACE
    for bad in (dict(page_size=128), dict(page_size=384), dict(pages_per_seq=0),
                dict(n_pages=0), dict(capacity=1000), dict(page_table=FAKE + 0x900002),
                dict(n_pages=1 << 22, page_size=512, pages_per_seq=2)):
        assert score(desc(**{**ok, **bad})) == INVALID, bad
    assert attn(desc(**{**ok, "v_stride_t": 256})) == INVALID    # V pool not in page layout
    assert attn(desc(**{**ok, "v_stride_h": 1000 * 128})) == INVALID


def test_baseline_comparator_validation():
    """K-means and dense-score comparators reject bad arguments before any launch."""
    d = desc()
    cbd = desc(codebook=FAKE + 0x500000)
    km = lib.sikv_kmeans_codebook
    need = lib.sikv_workspace_bytes(4, C.byref(cbd), 1, 1)
    assert need > 0 and lib.sikv_workspace_bytes(4, C.byref(d), 1, 1) == 0   # no codebook
    assert km(C.byref(d), FAKE, 0, 0, 128, 20, FAKE, need, None) == INVALID   # no codebook
    assert km(C.byref(cbd), None, 0, 0, 128, 20, FAKE, need, None) == INVALID
    assert km(C.byref(cbd), FAKE + 2, 0, 0, 128, 20, FAKE, need, None) == INVALID
    assert km(C.byref(cbd), FAKE, 0, 0, 100, 20, FAKE, need, None) == INVALID   # stride
    assert km(C.byref(cbd), FAKE, 0, 0, 128, 0, FAKE, need, None) == INVALID    # n_iter
    assert km(C.byref(cbd), FAKE, 0, 0, 128, 1001, FAKE, need, None) == INVALID
    assert km(C.byref(cbd), FAKE, 0, 0, 128, 20, FAKE, need - 8, None) == WORKSPACE
    assert km(C.byref(cbd), FAKE, 0, 0, 128, 20, None, 0, None) == WORKSPACE
    ds = lib.sikv_dense_scores
    assert ds(2, 2, 4, 1000, FAKE, FAKE, 0, 0, 128, None, None, None) == INVALID      # no output
    assert ds(2, 2, 3, 1000, FAKE, FAKE, 0, 0, 128, FAKE, None, None) == INVALID      # Hq % Hkv
    assert ds(2, 2, 18, 1000, FAKE, FAKE, 0, 0, 128, FAKE, None, None) == UNSUPPORTED  # G = 9
    assert ds(2, 2, 4, 0, FAKE, FAKE, 0, 0, 128, FAKE, None, None) == INVALID
    assert ds(2, 2, 4, 1000, FAKE + 2, FAKE, 0, 0, 128, FAKE, None, None) == INVALID
    assert ds(2, 2, 4, 1000, FAKE, FAKE, 0, 0, 100, FAKE, None, None) == INVALID     # stride
