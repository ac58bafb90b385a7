"""The C-ABI library on the CPU: it loads, exports every declared symbol, its
struct sizes match the binding, and host-side validation rejects bad
arguments before touching the device (no kernels are launched here)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "top_selected_attention.h")


@pytest.fixture(scope="module")
def tsa():
    import top_selected_attention_amd as t
    return t


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"TSA_API\s+[\w\s\*]+?\b(\w+)\s*\(", src)))


def test_every_declared_symbol_is_exported(tsa):
    names = _declared()
    assert len(names) >= 17
    for n in names:
        assert hasattr(tsa.lib, n), n
    assert set(names) == set(tsa._abi.EXPORTS)


def test_struct_sizes_match(tsa):
    for i, s in enumerate(tsa._abi.ARG_STRUCTS):
        assert tsa.lib.tsa_args_sizeof(i) == ctypes.sizeof(s)
    assert tsa.lib.tsa_args_sizeof(99) == 0


def test_status_strings(tsa):
    for code in range(7):
        assert tsa.lib.tsa_status_string(code)
    assert b"unknown" in tsa.lib.tsa_status_string(42)


def _bsa(tsa, **kw):
    a = dict(dtype=0, q_layout=0, kv_layout=0, B=2, N1=4, N2=2, Sq=1000, Skv=900, D=128,
             block_q=128, block_kv=64, sparse_mode=0, scale=0.088, validate=0, block_mask=16,
             q=16, k=16, v=16, out=16, lse=16)
    a.update(kw)
    return tsa._abi.BsaFwdArgs(**a)


def _size(tsa, fn, args):
    n = ctypes.c_size_t()
    return fn(ctypes.byref(args), ctypes.byref(n)), n.value


@pytest.mark.parametrize("kw,status", [
    (dict(), 0),
    (dict(D=64), 2),                       # headdim must be 128
    (dict(N1=3, N2=2), 2),                 # N1 % N2 != 0
    (dict(q_layout=1), 3),                 # q TND with k/v BNSD: mixed layouts not built
    (dict(q_layout=7), 2),
    (dict(sparse_mode=1), 2),
    (dict(dtype=5), 2),
    (dict(block_q=0), 2),
    (dict(q=0), 1),
    (dict(block_mask=0), 1),
    (dict(q=24), 2),                       # device tensors 16-byte aligned
    (dict(block_mask=8), 2),
    (dict(scale=float("nan")), 2),
    (dict(scale=0.0), 2),                  # scale must be positive
    (dict(scale=-0.1), 2),
    (dict(atten_mask=8), 0),               # atten_mask with shared planes
    (dict(atten_mask=8, atten_mask_stride_b=900000, atten_mask_stride_n=0), 0),
    (dict(atten_mask=8, atten_mask_stride_b=-1), 2),   # strides must be >= 0
    (dict(atten_mask=8, atten_mask_stride_n=-900000), 2),
    (dict(atten_mask=0, atten_mask_stride_n=-1), 0),    # no mask: strides ignored
    (dict(Sq=0), 0),                       # empty query: valid
    (dict(reuse_lists=1), 0),
    (dict(reuse_lists=2), 2),              # BSA has no partial-reuse mode
])
def test_bsa_validation(tsa, kw, status):
    s, n = _size(tsa, tsa.lib.bsa_fwd_workspace_size, _bsa(tsa, **kw))
    assert s == status
    if s == 0:
        assert n > 0


def _cu(*vals):
    return (ctypes.c_int32 * len(vals))(*vals)


@pytest.mark.parametrize("cq,ck,status", [
    ((0, 1000, 1700), (0, 900, 1500), 0),   # varlen, each sequence within Sq / Skv
    ((0, 1001, 1700), (0, 900, 1500), 2),   # a query sequence longer than Sq
    ((0, 1000, 1700), (0, 901, 1500), 2),   # a key sequence longer than Skv
    ((1, 1000, 1700), (0, 900, 1500), 2),   # prefix sums must start at 0
    ((0, 1000, 900), (0, 900, 1500), 2),    # and not decrease
    ((0, 0, 0), (0, 0, 0), 0),              # every sequence empty: valid
    (None, (0, 900, 1500), 1),              # TND needs both arrays
])
def test_bsa_tnd_validation(tsa, cq, ck, status):
    a = _bsa(tsa, q_layout=1, kv_layout=1)
    a.cu_seqlens_q = _cu(*cq) if cq else None
    a.cu_seqlens_kv = _cu(*ck)
    s, n = _size(tsa, tsa.lib.bsa_fwd_workspace_size, a)
    assert s == status
    if s == 0:
        assert n > 0
    b = tsa._abi.BsaBwdArgs(dtype=0, q_layout=1, kv_layout=1, B=2, N1=4, N2=2, Sq=1000,
                            Skv=900, D=128, block_q=128, block_kv=64, sparse_mode=2, scale=0.1,
                            block_mask=16, q=16, k=16, v=16, out=16, dout=16, lse=16, dq=16,
                            dk=16, dv=16)
    b.cu_seqlens_q, b.cu_seqlens_kv = a.cu_seqlens_q, a.cu_seqlens_kv
    assert _size(tsa, tsa.lib.bsa_bwd_workspace_size, b)[0] == status


def test_bsa_workspace_too_small_is_rejected_before_launch(tsa):
    a = _bsa(tsa)
    s, n = _size(tsa, tsa.lib.bsa_fwd_workspace_size, a)
    assert s == 0
    assert tsa.lib.bsa_fwd(ctypes.byref(a), ctypes.c_void_p(8), n - 1, None) == 4
    assert tsa.lib.bsa_fwd(ctypes.byref(a), None, n, None) == 4
    assert tsa.lib.bsa_fwd(None, None, 0, None) == 1


def test_bsa_bwd_validation(tsa):
    a = tsa._abi.BsaBwdArgs(dtype=0, q_layout=0, kv_layout=0, B=1, N1=2, N2=2, Sq=256, Skv=256,
                            D=128, block_q=128, block_kv=128, sparse_mode=2, scale=0.1,
                            block_mask=16, q=16, k=16, v=16, out=16, dout=16, lse=16, dq=16,
                            dk=16, dv=16)
    assert _size(tsa, tsa.lib.bsa_bwd_workspace_size, a)[0] == 0
    a.atten_mask, a.atten_mask_stride_b = 8, -5
    assert _size(tsa, tsa.lib.bsa_bwd_workspace_size, a)[0] == 2
    a.atten_mask_stride_b = 0
    assert _size(tsa, tsa.lib.bsa_bwd_workspace_size, a)[0] == 0
    a.dk = 0
    assert _size(tsa, tsa.lib.bsa_bwd_workspace_size, a)[0] == 1


def _nsa(tsa, seqlens=(256, 512), **kw):
    cu = (ctypes.c_int32 * (len(seqlens) + 1))(0, *[sum(seqlens[:i + 1]) for i in range(len(seqlens))])
    T = sum(seqlens)
    a = dict(dtype=0, layout=1, B=len(seqlens), T=T, Tk=T, N1=32, N2=2, D=128, Dv=128,
             cu_seqlens_q=ctypes.cast(cu, ctypes.POINTER(ctypes.c_int32)),
             cu_seqlens_kv=ctypes.cast(cu, ctypes.POINTER(ctypes.c_int32)),
             sbs=64, sbc=4, sparse_mode=2, scale=0.088, validate=0, topk=16, q=16, k=16, v=16,
             out=16, lse=16)
    a.update(kw)
    args = tsa._abi.NsaFwdArgs(**a)
    args._keep = cu
    return args


@pytest.mark.parametrize("kw,status", [
    (dict(), 0),
    (dict(layout=0), 3),                   # BNSD: only TND is supported
    (dict(sbs=8), 2),                      # block size a multiple of 16
    (dict(sbs=144), 2),                    # at most 128
    (dict(sbc=0), 2),
    (dict(sbc=129), 2),
    (dict(sbs=128, sbc=65), 2),            # product above 8K
    (dict(sparse_mode=1), 2),
    (dict(N1=31), 2),                      # N1 % N2
    (dict(N1=128, N2=2), 2),               # G = 64 > 32
    (dict(Dv=64), 3),                      # value heads other than 128 not built
    (dict(D=192), 0),                      # 192-dim query/key over 128-dim values
    (dict(D=64), 3),                       # other query/key dims not built
    (dict(T=100), 2),                      # cu_seqlens_q[B] != T
    (dict(topk=0), 1),
    (dict(v=40), 2),                       # device tensors 16-byte aligned
    (dict(reuse_lists=1), 0),
    (dict(reuse_lists=2), 2),              # the forward has no partial-reuse mode
])
def test_nsa_validation(tsa, kw, status):
    assert _size(tsa, tsa.lib.nsa_select_fwd_workspace_size, _nsa(tsa, **kw))[0] == status


@pytest.mark.parametrize("reuse,status,dq", [(0, 0, 16), (1, 0, 16), (2, 0, 16), (3, 2, 16),
                                             (-1, 2, 16), (0, 2, 20)])
def test_nsa_bwd_reuse_modes(tsa, reuse, status, dq):
    f = _nsa(tsa)
    fields = {n: getattr(f, n) for n, _ in f._fields_ if n not in ("out", "lse", "events")}
    fields.update(out=16, dout=16, lse=16, dq=dq, dk=16, dv=16, reuse_lists=reuse)
    b = tsa._abi.NsaBwdArgs(**fields)
    b._keep = f._keep
    assert _size(tsa, tsa.lib.nsa_select_bwd_workspace_size, b)[0] == status


def test_nsa_sequence_constraints(tsa):
    # a KV sequence shorter than sbs * sbc, and one not a multiple of sbs
    assert _size(tsa, tsa.lib.nsa_select_fwd_workspace_size, _nsa(tsa, seqlens=(192, 512)))[0] == 2
    assert _size(tsa, tsa.lib.nsa_select_fwd_workspace_size, _nsa(tsa, seqlens=(300, 512)))[0] == 2
    nb = ctypes.c_int32()
    assert tsa.lib.nsa_compact_blocks_total(ctypes.byref(_nsa(tsa)), ctypes.byref(nb)) == 0
    assert nb.value == (256 + 512) // 64


def test_nsa_list_calls_need_only_topk(tsa):
    """The list calls read shapes, cu_seqlens and topk: NULL attention tensors
    pass there and are refused by the forward."""
    a = _nsa(tsa, q=0, k=0, v=0, out=0, lse=0)
    assert _size(tsa, tsa.lib.nsa_compact_workspace_size, a)[0] == 0
    assert _size(tsa, tsa.lib.nsa_select_fwd_workspace_size, a)[0] == 1
    assert _size(tsa, tsa.lib.nsa_compact_workspace_size, _nsa(tsa, topk=0))[0] == 1


def _sfa(tsa, **kw):
    a = dict(dtype=0, q_layout=2, B=32, Sq=4, N1=64, N2=1, D=512, Dr=64, Dv=512,
             num_pages=16384, page_size=128, max_pages=512, topk=2048, sparse_block_size=1,
             sparse_mode=3, scale=1 / 24, validate=0, q=16, q_rope=16, key_cache=16,
             key_rope_cache=16, value_cache=16, block_table=16, kv_lens=16, topk_indices=16, out=16,
             lse=16)
    a.update(kw)
    return tsa._abi.SfaArgs(**a)


@pytest.mark.parametrize("cq,T,status", [
    ((0, 4, 9, 9), 9, 0),                  # ragged query counts, an empty entry
    ((0, 0, 0, 0), 0, 0),                  # no queries: valid
    ((1, 4, 9, 9), 9, 2),                  # prefix sums start at 0
    ((0, 4, 3, 9), 9, 2),                  # and do not decrease
    ((0, 4, 9, 9), 10, 2),                 # and end at T
])
def test_sfa_tnd_validation(tsa, cq, T, status):
    a = _sfa(tsa, q_layout=1, B=3, Sq=0, T=T)
    a.cu_seqlens_q = (ctypes.c_int32 * 4)(*cq)
    s, n = _size(tsa, tsa.lib.sfa_paged_fwd_workspace_size, a)
    assert s == status
    if s == 0:
        assert n > 0


@pytest.mark.parametrize("kw,status", [
    (dict(), 0),
    (dict(N1=48), 2),                      # N1 a power of two
    (dict(N1=256), 2),
    (dict(N2=2, N1=64), 3),                # one KV head only
    (dict(D=256), 2),
    (dict(Dr=32), 2),
    (dict(page_size=8), 2),
    (dict(page_size=2048), 2),
    (dict(sparse_block_size=3), 2),        # must divide the page size
    (dict(sparse_mode=2), 2),
    (dict(value_cache=32), 0),             # a value cache of its own
    (dict(value_cache=24), 2),             # (16-byte aligned)
    (dict(key_cache=24, value_cache=24), 2),   # caches 16-byte aligned
    (dict(q_rope=40), 2),
    (dict(q_layout=1), 1),                 # TND queries need cu_seqlens_q
    (dict(scale=0.0), 2),
    (dict(kv_lens=0), 1),
])
def test_sfa_validation(tsa, kw, status):
    assert _size(tsa, tsa.lib.sfa_paged_fwd_workspace_size, _sfa(tsa, **kw))[0] == status


def test_import_fails_loudly_without_library(tmp_path):
    """The binding has no fallback: without libtsa.so the import raises."""
    import shutil
    import subprocess
    import sys
    pkg = tmp_path / "top_selected_attention_amd"
    shutil.copytree(os.path.join(ROOT, "top_selected_attention_amd"), pkg,
                    ignore=shutil.ignore_patterns("*.so", "_build", "__pycache__"))
    r = subprocess.run([sys.executable, "-c", "import top_selected_attention_amd"],
                       cwd=tmp_path, capture_output=True, text=True)
    assert r.returncode != 0 and "libtsa.so" in r.stderr


def _skv(tsa, **kw):
    a = dict(dtype=0, q_layout=2, B=32, Sq=4, N1=64, N2=1, D=512, Dr=64, scale=1 / 24, q=16,
             q_rope=16, seqused_kv=16, has_ori_kv=1, has_cmp_kv=1, ori_win_left=127,
             ori_win_right=0, ori_num_pages=16384, ori_page_size=128, ori_max_pages=512,
             ori_key_cache=16, ori_key_rope_cache=16, ori_block_table=16, cmp_ratio=4,
             cmp_topk=512, cmp_num_pages=4096, cmp_page_size=128, cmp_max_pages=128,
             cmp_key_cache=16, cmp_key_rope_cache=16, cmp_block_table=16, cmp_topk_indices=16,
             out=16, lse=16)
    a.update(kw)
    return tsa._abi.SfaSharedkvArgs(**a)


@pytest.mark.parametrize("kw,status", [
    (dict(), 0),
    (dict(N1=48), 2),                          # N1 a power of two
    (dict(N2=2), 3),                           # one KV head
    (dict(D=256), 2),
    (dict(has_ori_kv=0, has_cmp_kv=0), 2),     # at least one branch
    (dict(has_ori_kv=2), 2),
    (dict(cmp_ratio=8), 2),                    # 4 or 128
    (dict(cmp_ratio=128), 0),
    (dict(cmp_topk=0), 2),
    (dict(ori_win_left=-1), 2),
    (dict(ori_win_left=4000, ori_win_right=100), 2),   # band of at most 4096 slots
    (dict(ori_page_size=8), 2),
    (dict(cmp_page_size=2048), 2),
    (dict(scale=0.0), 2),
    (dict(q=0), 1),
    (dict(cmp_topk_indices=0), 1),
    (dict(out=24), 2),                         # device tensors 16-byte aligned
    (dict(cmp_key_rope_cache=8), 2),
    (dict(has_cmp_kv=0, cmp_key_cache=0, cmp_topk_indices=0, cmp_ratio=0), 0),
    (dict(has_ori_kv=0, ori_key_cache=0, ori_block_table=0, ori_win_left=-5), 0),
    (dict(q_layout=1, T=128), 1),              # TND needs cu_seqlens_q
    (dict(B=0), 0),                            # no tokens
])
def test_sfa_sharedkv_validation(tsa, kw, status):
    s, n = _size(tsa, tsa.lib.sfa_sharedkv_fwd_workspace_size, _skv(tsa, **kw))
    assert s == status
    if s == 0:
        assert n > 0


def test_sfa_sharedkv_workspace_too_small_is_rejected_before_launch(tsa):
    a = _skv(tsa)
    s, n = _size(tsa, tsa.lib.sfa_sharedkv_fwd_workspace_size, a)
    assert s == 0
    assert tsa.lib.sfa_sharedkv_fwd(ctypes.byref(a), ctypes.c_void_p(8), n - 1, None) == 4
    # large enough but not 16-byte aligned
    assert tsa.lib.sfa_sharedkv_fwd(ctypes.byref(a), ctypes.c_void_p(24), n + 64, None) == 4



def test_sfa_sharedkv_metadata_size_and_buffer_checks(tsa):
    a = _skv(tsa)
    n = ctypes.c_size_t()
    assert tsa.lib.sfa_sharedkv_metadata_size(ctypes.byref(a), ctypes.byref(n)) == 0
    # 128 tokens: prefix sums (padded) + 4 ints of token entry + 2 per split range
    assert n.value % 4 == 0 and n.value >= 4 * (36 + 128 * 4 + 128 * 2)
    assert tsa.lib.sfa_sharedkv_metadata(ctypes.byref(a), ctypes.c_void_p(8), n.value - 4,
                                         None) == 4
    assert tsa.lib.sfa_sharedkv_metadata(ctypes.byref(a), None, n.value, None) == 4
    # a task list off a 16-byte boundary is refused before any launch
    assert tsa.lib.sfa_sharedkv_metadata(ctypes.byref(a), ctypes.c_void_p(8), n.value, None) == 2
    w = ctypes.c_size_t()
    assert tsa.lib.sfa_sharedkv_fwd_workspace_size(ctypes.byref(a), ctypes.byref(w)) == 0
    a.tasks = 24
    assert tsa.lib.sfa_sharedkv_fwd(ctypes.byref(a), ctypes.c_void_p(256), w.value, None) == 2
    bad = _skv(tsa, N1=48)
    assert tsa.lib.sfa_sharedkv_metadata_size(ctypes.byref(bad), ctypes.byref(n)) == 2


def _floyd(tsa, bwd=False, **kw):
    a = dict(dtype=0, B=1, H=2, N=16, M=128, K=128, D=64, scale=0.125, q=256, k1=512, v1=768,
             k2=1024, v2=1280, out=1536, lse=1792)
    if bwd:
        a.update(dout=2048, dq=2304, dk1=2560, dv1=2816, dk2=3072, dv2=3328)
    a.update(kw)
    return (tsa._abi.FloydBwdArgs if bwd else tsa._abi.FloydFwdArgs)(**a)


@pytest.mark.parametrize("kw,status", [
    ({}, 0),
    (dict(N=24), 2),                       # N a multiple of 16
    (dict(N=0), 2),
    (dict(M=192), 2),                      # M a multiple of 128
    (dict(K=64), 2),                       # K at least 128
    (dict(D=48), 2),                       # D in {32, 64, 128}
    (dict(H=257), 2),
    (dict(B=2049), 2),
    (dict(scale=0.0), 2),
    (dict(dtype=3), 2),
    (dict(k2=0), 1),
    (dict(v1=264), 2),                     # 16-byte aligned tensors
])
def test_floyd_validation(tsa, kw, status):
    assert _size(tsa, tsa.lib.floyd_fwd_workspace_size, _floyd(tsa, **kw))[0] == status
    assert _size(tsa, tsa.lib.floyd_bwd_workspace_size, _floyd(tsa, True, **kw))[0] == status


def test_floyd_workspace_sizes(tsa):
    """fp32 S + 16-bit P + fp32 [rows, D] forward; the backward adds fp32 dP
    and a 16-bit dS (each B*H*N*M*K elements)."""
    s, f = _size(tsa, tsa.lib.floyd_fwd_workspace_size, _floyd(tsa))
    s2, b = _size(tsa, tsa.lib.floyd_bwd_workspace_size, _floyd(tsa, True))
    el, rows = 2 * 16 * 128 * 128, 2 * 16 * 128
    assert s == s2 == 0
    assert el * 6 + rows * 64 * 4 <= f <= el * 6 + rows * 64 * 4 + 4096
    assert el * 12 + rows * 64 * 4 <= b <= el * 12 + rows * 64 * 4 + 4096
    assert _size(tsa, tsa.lib.floyd_bwd_workspace_size, _floyd(tsa, True, dq=0))[0] == 1
