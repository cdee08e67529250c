"""C ABI checks that need no GPU: exports, status strings, workspace sizing,
and argument validation (every error returns before anything is enqueued)."""
import ctypes
import os
import re

import pytest

from chunked_kl_loss_row_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="libkdchunk.so not built")


def _has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(kd_[a-z_0-9]+)\s*\(", text, re.M))
    return sorted(names)


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(B.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for st in range(8):
        s = B.kd_status_string(st)
        assert s.startswith("KD_OK" if st == 0 else "KD_ERR_")
    assert "unknown" in B.kd_status_string(99)


def P(n=1000, d=128, v=4096, k=16, chunk=64, x=B.KD_BF16, t=None, tau=1.0, dw_chunks=1):
    return B.problem(n, d, v, k, chunk, x, t, tau, dw_chunks)


def test_workspace_independent_of_n():
    sizes = {B.kd_chunked_workspace_size(P(n=n)) for n in (0, 1, 64, 1000, 10 ** 9)}
    assert len(sizes) == 1 and sizes.pop() > 0


def test_workspace_grows_with_chunk_and_dtype():
    a = B.kd_chunked_workspace_size(P(chunk=64))
    b = B.kd_chunked_workspace_size(P(chunk=128))
    c = B.kd_chunked_workspace_size(P(chunk=64, x=B.KD_F32))
    assert a < b and a < c
    # the chunk's dZ tile (chunk x padded V) dominates: at least chunk * V * 2 bytes
    big = B.kd_chunked_workspace_size(P(n=32768, d=2880, v=201088, k=100, chunk=2048))
    assert 2048 * 201088 * 2 <= big < 2 * 2048 * 201088 * 2


@pytest.mark.parametrize("kw", [dict(n=-1), dict(d=0), dict(v=0), dict(k=0), dict(k=257, v=1000),
                                dict(k=20, v=10), dict(chunk=0), dict(v=16777216),
                                dict(d=65544), dict(tau=-1.0), dict(tau=0.005), dict(tau=101.0),
                                dict(tau=float("nan")), dict(tau=float("inf")), dict(dw_chunks=-1),
                                dict(dw_chunks=9)])
def test_bad_shapes(kw):
    prob = P(**kw)
    assert B.kd_chunked_workspace_size(prob) == 0
    st = B.kd_chunked_fwd(prob, 16, 16, 16, 16, None, 16, 16, workspace=16, workspace_bytes=1 << 40,
                          stream=0, check=False)
    assert st == B.KD_ERR_SHAPE


def test_bad_dtype_and_alignment():
    fake = 1 << 20
    for prob, want in ((P(x=2), B.KD_ERR_DTYPE), (P(t=7), B.KD_ERR_DTYPE), (P(d=12), B.KD_ERR_ALIGN)):
        st = B.kd_chunked_fwd(prob, fake, fake, fake, fake, None, fake, fake, workspace=fake,
                              workspace_bytes=1 << 40, stream=0, check=False)
        assert st == want
    st = B.kd_chunked_fwd(P(), fake + 2, fake, fake, fake, None, fake, fake, workspace=fake,
                          workspace_bytes=1 << 40, stream=0, check=False)
    assert st == B.KD_ERR_ALIGN
    st = B.kd_chunked_bwd(P(), fake, fake, fake, fake, None, fake, None, fake + 4, fake,
                          workspace=fake, workspace_bytes=1 << 40, stream=0, check=False)
    assert st == B.KD_ERR_ALIGN
    # dW is read and written 16 bytes at a time
    st = B.kd_chunked_bwd(P(), fake, fake, fake, fake, None, fake, None, fake, fake + 4,
                          workspace=fake, workspace_bytes=1 << 40, stream=0, check=False)
    assert st == B.KD_ERR_ALIGN


def test_null_pointers():
    fake = 1 << 20
    st = B.lib().kd_chunked_fwd(None, fake, fake, fake, fake, None, fake, fake, None, None, fake, 1 << 40, None)
    assert st == B.KD_ERR_NULL
    args = dict(H=fake, W=fake, t_ids=fake, t_logits=fake, lse=fake)
    for missing in args:
        a = dict(args)
        a[missing] = None
        st = B.kd_chunked_fwd(P(), a["H"], a["W"], a["t_ids"], a["t_logits"], None, fake, a["lse"],
                              workspace=fake, workspace_bytes=1 << 40, stream=0, check=False)
        assert st == B.KD_ERR_NULL, missing
    st = B.kd_chunked_fwd(P(), fake, fake, fake, fake, None, None, fake, workspace=fake,
                          workspace_bytes=1 << 40, stream=0, check=False)
    assert st == B.KD_ERR_NULL
    st = B.kd_chunked_bwd(P(), fake, fake, fake, fake, None, fake, None, fake, None, workspace=fake,
                          workspace_bytes=1 << 40, stream=0, check=False)
    assert st == B.KD_ERR_NULL


def test_workspace_too_small():
    fake = 1 << 20
    need = B.kd_chunked_workspace_size(P())
    st = B.kd_chunked_fwd(P(), fake, fake, fake, fake, None, fake, fake, workspace=fake,
                          workspace_bytes=need - 1, stream=0, check=False)
    assert st == B.KD_ERR_WORKSPACE
    st = B.kd_chunked_bwd(P(), fake, fake, fake, fake, None, fake, None, fake, fake, workspace=fake,
                          workspace_bytes=need - 1, stream=0, check=False)
    assert st == B.KD_ERR_WORKSPACE


@pytest.mark.skipif(_has_gpu(), reason="with a GPU present valid arguments would launch")
def test_valid_arguments_without_gpu_report_device():
    fake = 1 << 20
    need = B.kd_chunked_workspace_size(P())
    st = B.kd_chunked_fwd(P(), fake, fake, fake, fake, None, fake, fake, workspace=fake,
                          workspace_bytes=need, stream=0, check=False)
    assert st == B.KD_ERR_DEVICE
    with pytest.raises(B.KDError):
        B.kd_chunked_bwd(P(), fake, fake, fake, fake, None, fake, None, fake, fake, workspace=fake,
                         workspace_bytes=need, stream=0)


def test_validate_argument_errors():
    fake = 1 << 20
    st = B.kd_chunked_validate(P(), fake, None, None, stream=0, check=False)
    assert st == B.KD_ERR_NULL
    st = B.kd_chunked_validate(P(), None, None, fake, stream=0, check=False)
    assert st == B.KD_ERR_NULL
    st = B.kd_chunked_validate(P(), fake, None, fake + 4, stream=0, check=False)
    assert st == B.KD_ERR_ALIGN
    st = B.kd_chunked_validate(P(k=0), fake, None, fake, stream=0, check=False)
    assert st == B.KD_ERR_SHAPE
    st = B.kd_chunked_validate(P(n=4 * 2 ** 31), fake, None, fake, stream=0, check=False)
    assert st == B.KD_ERR_SHAPE
    if not _has_gpu():
        assert B.kd_chunked_validate(P(), fake, None, fake, stream=0, check=False) == B.KD_ERR_DEVICE


def test_profile_hook_without_launches():
    assert B.kd_profile_enable(True) == 0
    allk = B.kd_profile_all()
    assert len(allk) == B.KD_K_COUNT and all(v == (0.0, 0) for v in allk.values())
    assert "fwd_proj" in allk and "bwd_dw" in allk
    with pytest.raises(B.KDError):
        B.kd_profile_read(B.KD_K_COUNT)
    assert B.kd_profile_enable(False) == 0


def test_tile_offset_limits():
    # 256 rows of the padded vocabulary (dZ) or of the rounded chunk (H_c^T)
    # must stay below 2^31 bytes: the largest accepted sizes and one beyond
    for x, vmax, cmax in ((B.KD_BF16, 4194048, 4194296), (B.KD_F32, 2097024, 2097144)):
        assert B.kd_chunked_workspace_size(P(v=vmax, x=x, k=4, chunk=4)) > 0
        assert B.kd_chunked_workspace_size(P(v=vmax + 1, x=x, k=4, chunk=4)) == 0
        assert B.kd_chunked_workspace_size(P(chunk=cmax, x=x)) > 0
        assert B.kd_chunked_workspace_size(P(chunk=cmax + 1, x=x)) == 0


def test_projection_tile_count_limit():
    # a chunk's projection grid (512 work-items per 256 x 384 tile) must stay
    # below 2^32 work-items: at most 8388600 tiles
    v = 4194048                                   # 10922 vocabulary tiles
    assert B.kd_chunked_workspace_size(P(v=v, k=4, chunk=768 * 256)) > 0          # 8388096 tiles
    assert B.kd_chunked_workspace_size(P(v=v, k=4, chunk=768 * 256 + 1)) == 0      # 8399018 tiles
    assert B.kd_teacher_topk_workspace_size(P(v=v, k=4, chunk=768 * 256 + 1)) == 0


def test_temperature_zero_reads_as_one():
    assert B.kd_chunked_workspace_size(P(tau=0.0)) == B.kd_chunked_workspace_size(P(tau=1.0)) > 0
    assert B.kd_chunked_workspace_size(P(tau=0.01)) > 0 and B.kd_chunked_workspace_size(P(tau=100.0)) > 0


def test_problem_struct_layout():
    # int64 n, six int32 fields, float tau, int32 dw_chunks
    assert ctypes.sizeof(B.KDProblem) == 40 and B.KDProblem.tau.offset == 32
    assert B.KDProblem.dw_chunks.offset == 36


def test_dw_chunks_workspace():
    one = B.kd_chunked_workspace_size(P(dw_chunks=1))
    assert B.kd_chunked_workspace_size(P(dw_chunks=0)) == one
    two = B.kd_chunked_workspace_size(P(dw_chunks=2))
    big = B.problem(32768, 2880, 201088, 100, 2048, B.KD_BF16, None, 1.0, 2)
    dz = 2048 * 201216 * 2  # one chunk of dZ at the gpt-oss shapes
    assert two > one
    assert B.kd_chunked_workspace_size(big) - B.kd_chunked_workspace_size(P(32768, 2880, 201088, 100, 2048)) >= dz
    # the transposed H of a group also counts against the 32-bit tile limit
    assert B.kd_chunked_workspace_size(P(chunk=2097148, dw_chunks=2)) > 0
    assert B.kd_chunked_workspace_size(P(chunk=2097149, dw_chunks=2)) == 0


def test_noalloc_forward_argument_errors():
    """kd_chunked_fwd_noalloc checks its arguments like kd_chunked_fwd, and
    refuses a problem whose chunk does not fit the library's scratch."""
    fake = 1 << 20
    lib = B.lib()
    assert lib.kd_chunked_fwd_noalloc(None, fake, fake, fake, fake, None, fake, fake, None, None, None) == \
        B.KD_ERR_NULL
    assert B.kd_chunked_fwd_noalloc(P(k=0), fake, fake, fake, fake, None, fake, fake, stream=0,
                                    check=False) == B.KD_ERR_SHAPE
    assert B.kd_chunked_fwd_noalloc(P(), fake, fake, fake, fake, None, None, fake, stream=0,
                                    check=False) == B.KD_ERR_NULL
    assert B.kd_chunked_fwd_noalloc(P(), fake, None, fake, fake, None, fake, fake, stream=0,
                                    check=False) == B.KD_ERR_NULL
    assert B.kd_chunked_fwd_noalloc(P(), fake + 8, fake, fake, fake, None, fake, fake, stream=0,
                                    check=False) == B.KD_ERR_ALIGN
    # one 2048-row chunk of the 32K gpt-oss shapes fits (about 25 MB); 8192 rows do not
    big = dict(n=32768, d=2880, v=201088, k=100)
    st_fit = B.kd_chunked_fwd_noalloc(P(chunk=2048, **big), fake, fake, fake, fake, None, fake, fake,
                                      stream=0, check=False)
    assert st_fit != B.KD_ERR_WORKSPACE
    assert B.kd_chunked_fwd_noalloc(P(chunk=8192, **big), fake, fake, fake, fake, None, fake, fake,
                                    stream=0, check=False) == B.KD_ERR_WORKSPACE
    if not _has_gpu():
        assert st_fit == B.KD_ERR_DEVICE
    # the oversized problem the GPU test uses is refused on the host
    assert B.kd_chunked_fwd_noalloc(B.problem(64, 8192, 200000, 100, 4096, B.KD_BF16), fake, fake, fake, fake,
                                    None, fake, fake, stream=0, check=False) == B.KD_ERR_WORKSPACE


def test_noalloc_scratch_size_matches_header():
    text = open(os.path.join(ROOT, "include", "kd_chunked.h")).read()
    m = re.search(r"#define KD_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == B.NOALLOC_SCRATCH_BYTES
