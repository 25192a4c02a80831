"""The C-ABI library without a GPU: it loads, exports every declared entry
point, and its static validation returns the documented codes before any
device query."""
import ctypes
import os
import re

import pytest

import beta_epilogue_amd as ge

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm_epi.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_epi_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(ge.LIB_PATH)
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), "missing export " + n


def test_measurement_library_exports_its_declared_symbol():
    """libmfma_ceiling.so (bench.py --mfma-ceiling) exports what
    include/mfma_ceiling.h declares."""
    text = open(os.path.join(ROOT, "include", "mfma_ceiling.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(mfma_ceiling_\w+)\s*\(", text)))
    assert names == ["mfma_ceiling_run", "mfma_ceiling_run_type"]
    lib = ctypes.CDLL(os.path.join(ROOT, "beta_epilogue_amd", "libmfma_ceiling.so"))
    for n in names:
        assert hasattr(lib, n), "missing export " + n


def test_status_strings():
    assert ge.status_string(0) == "success"
    for c in range(1, 7):
        assert ge.status_string(c) not in ("success", "unknown status")
    assert ge.status_string(99) == "unknown status"


def test_variant_table():
    n = ge.gemm_epi_variant_count()
    assert n >= 10
    names = [ge.gemm_epi_variant_name(i) for i in range(n)]
    assert len(set(names)) == n
    assert ge.gemm_epi_variant_name(-1) is None and ge.gemm_epi_variant_name(n) is None


def _create(**kw):
    base = dict(M=256, N=256, K=256, L=1, ab="f16", c="f16", x="f16", d="f16", y="f16")
    base.update(kw)
    M, N, K, L = base.pop("M"), base.pop("N"), base.pop("K"), base.pop("L")
    desc = ge.make_desc(M, N, K, L, **base)
    h = ctypes.c_void_p(1234)
    rc = ge.lib().gemm_epi_create(ctypes.byref(desc), ctypes.byref(h))
    return rc, h.value


BAD = [
    (dict(M=0), ge.GEMM_EPI_ERR_INVALID_ARG),
    (dict(K=-8), ge.GEMM_EPI_ERR_INVALID_ARG),
    (dict(L=0), ge.GEMM_EPI_ERR_INVALID_ARG),
    (dict(M=2**40, N=2**40), ge.GEMM_EPI_ERR_INVALID_ARG),       # int64 overflow
    (dict(ab="f32"), ge.GEMM_EPI_ERR_INVALID_ARG),                # not an A/B type
    (dict(ab="i8"), ge.GEMM_EPI_ERR_UNSUPPORTED),                 # int8 needs int32 outs
    (dict(ab="f16", d="i32"), ge.GEMM_EPI_ERR_UNSUPPORTED),
    (dict(ab="f16", c="e4m3"), ge.GEMM_EPI_ERR_UNSUPPORTED),
    (dict(ab="e5m2", d="e5m2"), ge.GEMM_EPI_ERR_UNSUPPORTED),     # fp8 is A/B only
    (dict(d=None), ge.GEMM_EPI_ERR_UNSUPPORTED),                  # D required
    (dict(K=100), ge.GEMM_EPI_ERR_ALIGNMENT),                     # 200 B rows
    (dict(N=100), ge.GEMM_EPI_ERR_ALIGNMENT),                     # f16 C/D rows
    (dict(ab="e4m3", K=8), ge.GEMM_EPI_ERR_ALIGNMENT),            # 8 B rows
    (dict(a_major="M", M=100), ge.GEMM_EPI_ERR_ALIGNMENT),
    (dict(M=16, N=2**21, K=64), ge.GEMM_EPI_ERR_UNSUPPORTED),    # 31-bit epilogue offsets
    (dict(splits=-1), ge.GEMM_EPI_ERR_INVALID_ARG),
    (dict(ab="u8"), ge.GEMM_EPI_ERR_UNSUPPORTED),                 # uint8 needs int32 outs
    (dict(ab="u8", b="i8", c="i32", x="i32", d="i32", y="i32"), ge.GEMM_EPI_ERR_INVALID_ARG),
    (dict(ab="u8", c="i32", x="i32", d="i32", y="i32", a_major="M", M=8), ge.GEMM_EPI_ERR_ALIGNMENT),
]


@pytest.mark.parametrize("kw,code", BAD, ids=[str(b[0]) for b in BAD])
def test_create_static_validation(kw, code):
    rc, h = _create(**kw)
    assert rc == code, (rc, ge.last_error())
    assert h is None  # *out cleared on error
    assert ge.last_error()


def test_create_bad_enums():
    desc = ge.make_desc(256, 256, 256, 1, ab="f16", d="f16")
    desc.a_major = 2  # 'N' is not a majorness of A
    h = ctypes.c_void_p()
    assert ge.lib().gemm_epi_create(ctypes.byref(desc), ctypes.byref(h)) == \
        ge.GEMM_EPI_ERR_INVALID_ARG
    desc = ge.make_desc(256, 256, 256, 1, ab="f16", d="f16")
    desc.d_dtype = 17
    assert ge.lib().gemm_epi_create(ctypes.byref(desc), ctypes.byref(h)) == \
        ge.GEMM_EPI_ERR_INVALID_ARG
    desc = ge.make_desc(256, 256, 256, 1, ab="f16", d="f16", b="e5m2")
    assert ge.lib().gemm_epi_create(ctypes.byref(desc), ctypes.byref(h)) == \
        ge.GEMM_EPI_ERR_INVALID_ARG  # only the fp8 formats pair
    desc = ge.make_desc(256, 256, 256, 1, ab="f16", d="f16")
    desc.epilogue = 2  # only LINEAR (0) and RELU (1)
    assert ge.lib().gemm_epi_create(ctypes.byref(desc), ctypes.byref(h)) == \
        ge.GEMM_EPI_ERR_INVALID_ARG
    assert "epilogue" in ge.last_error()
    assert ge.lib().gemm_epi_create(None, ctypes.byref(h)) == ge.GEMM_EPI_ERR_INVALID_ARG
    assert ge.lib().gemm_epi_create(ctypes.byref(desc), None) == ge.GEMM_EPI_ERR_INVALID_ARG


def test_mixed_epilogue_types_run_on_every_block_shape():
    """Mixed C/X/D/Y types (the general epilogue) are accepted by 16x16- and
    32x32-block variants alike: validation passes and, with no GPU here,
    creation stops at the device query."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    names = [ge.gemm_epi_variant_name(i) for i in range(ge.gemm_epi_variant_count())]
    for v, cd in (("bf16_kk_n_256x256_r128_w4_s2_b16", "N"), ("bf16_kk_m_256x256_r128_w4_s2_q2", "M")):
        desc = ge.make_desc(304, 264, 128, 1, ab="bf16", c="f32", x="bf16", d="f32", cd_major=cd)
        h = ctypes.c_void_p()
        assert ge.lib().gemm_epi_create_variant(ctypes.byref(desc), names.index(v),
                                                ctypes.byref(h)) == ge.GEMM_EPI_ERR_DEVICE
        assert h.value is None


def test_fp8_with_fp32_outputs_only_widened():
    """fp8 A/B with an fp32 D or Y run widened: an fp16 kernel of the layout
    on fp16 copies of A and B.  An fp8-MFMA variant refuses such a problem,
    the fp16 one accepts it; without fp32 outputs the fp8 kernel of the
    pairing runs and the fp16 one is refused, unless the pairing has no fp8
    kernel for the layout (then the fp16 one runs it)."""
    names = [ge.gemm_epi_variant_name(i) for i in range(ge.gemm_epi_variant_count())]
    f8 = names.index("e4m3_kk_n_256x256_r128_w4_s2")
    e45 = names.index("e4e5_kk_n_256x256_r128_w4_s2")
    f16 = names.index("f16_kk_n_256x256_r128_w4_s2_b16")
    f16_mn = names.index("f16_mn_n_256x256_r128_w4_s2_q2")
    h = ctypes.c_void_p()
    cases = (("f32", None, f8, False, None, "K", "K"), ("f16", "f32", f8, False, None, "K", "K"),
             ("f32", None, f16, True, None, "K", "K"), ("f16", "f32", f16, True, None, "K", "K"),
             ("f16", None, f16, False, None, "K", "K"), ("f16", None, f8, True, None, "K", "K"),
             ("f16", None, e45, True, "e5m2", "K", "K"), ("f16", None, f16, False, "e5m2", "K", "K"),
             ("f16", None, f8, False, "e5m2", "K", "K"),
             # the e4m3 x e5m2 pairing has no fp8 kernel with M-major A and N-major B
             ("f16", None, f16_mn, True, "e5m2", "M", "N"))
    for d, y, v, ok, b, am, bm in cases:
        desc = ge.make_desc(256, 256, 256, 1, ab="e4m3", c="f16", d=d, y=y, b=b, a_major=am, b_major=bm)
        rc = ge.lib().gemm_epi_create_variant(ctypes.byref(desc), v, ctypes.byref(h))
        if ok:
            assert rc in (ge.GEMM_EPI_OK, ge.GEMM_EPI_ERR_DEVICE), (d, y, names[v])
            if h.value:
                ge.lib().gemm_epi_destroy(h)
        else:
            assert rc == ge.GEMM_EPI_ERR_UNSUPPORTED, (d, y, names[v], rc)


def test_every_majorness_has_a_kernel():
    """Every A/B type with every A ('K', 'M'), B ('K', 'N') and C/D ('N', 'M')
    majorness is accepted by static validation (with no GPU here, creation
    stops at the device query, never at "no kernel")."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    for ab, b, outs in (("f16", None, "f16"), ("bf16", None, "f32"), ("e4m3", None, "f16"),
                        ("e5m2", None, "f16"), ("e4m3", "e5m2", "f16"), ("e5m2", "e4m3", "f32"),
                        ("i8", None, "i32"), ("u8", None, "i32")):
        for a_major in "KM":
            for b_major in "KN":
                for cd in "NM":
                    rc, h = _create(ab=ab, b=b, a_major=a_major, b_major=b_major, cd_major=cd,
                                    c=outs, x=None, d=outs, y=None)
                    assert rc == ge.GEMM_EPI_ERR_DEVICE, (ab, b, a_major, b_major, cd, rc,
                                                          ge.last_error())


def test_too_large_mn_major_operand_is_an_error_not_a_fallback():
    """An M-major A beyond 2 GiB per batch cannot be addressed with the
    kernels' 32-bit offsets: refused at create, before any device query."""
    rc, _ = _create(a_major="M", M=65536, K=32768, N=16)
    assert rc == ge.GEMM_EPI_ERR_UNSUPPORTED, ge.last_error()
    assert "2 GiB" in ge.last_error()


def test_run_and_plan_reject_null_handle():
    assert ge.lib().gemm_epi_run(None, 16, 16, None, None, 16, None, 1.0, 0.0, 0.0,
                                 None) == ge.GEMM_EPI_ERR_INVALID_ARG
    p = ge.gemm_epi_plan()
    assert ge.lib().gemm_epi_get_plan(None, ctypes.byref(p)) == ge.GEMM_EPI_ERR_INVALID_ARG
    assert ge.lib().gemm_epi_destroy(None) == ge.GEMM_EPI_OK


def test_valid_problem_needs_a_device_here():
    """With no GPU, a valid problem passes validation and stops at the device
    query (never a silent CPU path)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    rc, h = _create()
    assert rc == ge.GEMM_EPI_ERR_DEVICE and h is None


def test_product_does_not_reference_the_oracle():
    """The product package never imports or links the oracle."""
    pkg = os.path.join(ROOT, "beta_epilogue_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f
