"""The C-ABI library loads, exports every symbol its header declares, and
rejects invalid arguments on the host, before any device work (CPU only)."""

import ctypes
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mha.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mha_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("mha_create", "mha_workspace_size", "mha_forward", "mha_destroy",
                     "mha_status_string"):
        assert required in names


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_header_is_plain_c99():
    src = '#include "mha.h"\nint main(void) { return MHA_OK; }\n'
    p = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic", "-fsyntax-only",
                        "-I", os.path.join(ROOT, "include"), "-x", "c", "-"],
                       input=src, text=True, capture_output=True)
    assert p.returncode == 0, p.stderr


@pytest.fixture(scope="module")
def mha():
    import transformer_head_attention_amd as m
    return m


def test_library_exports_every_declared_symbol(mha):
    lib = ctypes.CDLL(mha.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert set(mha.EXPORTED) == set(_declared_functions())


def test_status_and_stage_strings(mha):
    for s in range(5):
        assert mha.mha_status_string(s).startswith("MHA_")
    assert [mha.mha_stage_name(i) for i in range(mha.MHA_NUM_STAGES)] == \
        ["prep", "qkv_proj", "attention", "out_proj", "early_rows"]
    assert mha.mha_stage_name(mha.MHA_NUM_STAGES) is None


def test_create_validation(mha):
    st, h = mha.mha_create(512, 7, mha.MHA_BF16)          # not divisible
    assert st == mha.MHA_ERR_INVALID_ARG and h is None
    st, h = mha.mha_create(512, 0, mha.MHA_BF16)
    assert st == mha.MHA_ERR_INVALID_ARG
    st, h = mha.mha_create(256, 8, mha.MHA_BF16)          # d_k = 32
    assert st == mha.MHA_ERR_UNSUPPORTED
    st, h = mha.mha_create(32, 8, mha.MHA_F32)            # the d_v = 4 example: oracle only
    assert st == mha.MHA_ERR_UNSUPPORTED
    st, h = mha.mha_create(192, 3, mha.MHA_BF16)          # d_k 64 but D % 128 != 0
    assert st == mha.MHA_ERR_UNSUPPORTED
    st, h = mha.mha_create(512, 8, 7)
    assert st == mha.MHA_ERR_INVALID_ARG
    for D, heads, dt in ((512, 8, mha.MHA_F32), (1024, 16, mha.MHA_BF16), (4096, 32, mha.MHA_BF16)):
        st, h = mha.mha_create(D, heads, dt)
        assert st == mha.MHA_OK and h
        assert mha.mha_destroy(h) == mha.MHA_OK
    assert mha.mha_destroy(None) == mha.MHA_OK


def test_workspace_size(mha):
    st, h = mha.mha_create(1024, 16, mha.MHA_BF16)
    try:
        n = mha.mha_workspace_size(h, 8, 4096, 4096)
        assert n > 0 and n % 256 == 0
        # Q, K, V^T, O in fp16 plus the transposed weights dominate
        assert n >= 4 * 8 * 4096 * 1024 * 2 + 4 * 1024 * 1024 * 2
        assert mha.mha_workspace_size(h, 0, 4096, 4096) == 0
        assert mha.mha_workspace_size(h, 8, 0, 4096) == 0
        assert mha.mha_workspace_size(None, 8, 4096, 4096) == 0
        assert mha.mha_workspace_size(h, 2, 100, 300) < mha.mha_workspace_size(h, 2, 100, 600)
        # d_k = 64: a key/value set's K block must stay below 2 GiB (32-bit offsets)
        assert mha.mha_workspace_size(h, 1, 64, (1 << 24) - 256) > 0
        assert mha.mha_workspace_size(h, 1, 64, (1 << 24) + 1) == 0
    finally:
        mha.mha_destroy(h)


def test_forward_rejects_bad_arguments_before_device_work(mha):
    st, h = mha.mha_create(512, 8, mha.MHA_BF16)
    fake = 1 << 20          # aligned dummy addresses: never dereferenced on these paths
    ws = mha.mha_workspace_size(h, 2, 16, 16)

    def call(**kw):
        args = dict(x_q=fake, x_kv=None, w_qkv=fake, b_qkv=None, w_o=fake, b_o=None, B=2,
                    T_q=16, T_k=16, causal=0, key_padding_mask=None, y=fake, workspace=fake,
                    workspace_bytes=ws, stream=None)
        args.update(kw)
        return mha.mha_forward(h, *args.values())

    try:
        assert mha.mha_forward(None, fake, None, fake, None, fake, None, 2, 16, 16, 0, None,
                               fake, fake, ws, None) == mha.MHA_ERR_INVALID_ARG
        assert call(x_q=None) == mha.MHA_ERR_INVALID_ARG
        assert call(y=None) == mha.MHA_ERR_INVALID_ARG
        assert call(causal=2) == mha.MHA_ERR_INVALID_ARG
        assert call(T_k=20) == mha.MHA_ERR_INVALID_ARG               # self-attention, T_k != T_q
        assert call(x_kv=fake, T_k=20, causal=1) == mha.MHA_ERR_INVALID_ARG
        assert call(B=0) == mha.MHA_ERR_INVALID_ARG
        assert call(x_q=fake + 2) == mha.MHA_ERR_INVALID_ARG          # misaligned
        assert call(workspace_bytes=ws - 1) == mha.MHA_ERR_WORKSPACE
    finally:
        mha.mha_destroy(h)


def test_profile_calls_validate(mha):
    st, h = mha.mha_create(512, 8, mha.MHA_BF16)
    try:
        assert mha.mha_profile_begin(h, 0) == mha.MHA_ERR_INVALID_ARG
        assert mha.mha_profile_begin(None, 4) == mha.MHA_ERR_INVALID_ARG
    finally:
        mha.mha_destroy(h)


def test_create_grouped_validation_and_workspace(mha):
    for n_g in (0, -1, 3, 5, 32):                          # < 1 or not dividing 16
        st, h = mha.mha_create_grouped(1024, 16, n_g, mha.MHA_BF16)
        assert st == mha.MHA_ERR_INVALID_ARG and h is None
    st, h = mha.mha_create_grouped(256, 8, 2, mha.MHA_BF16)   # d_k = 32
    assert st == mha.MHA_ERR_UNSUPPORTED
    sizes = {}
    for n_g in (16, 4, 1):
        st, h = mha.mha_create_grouped(1024, 16, n_g, mha.MHA_BF16)
        assert st == mha.MHA_OK and h
        sizes[n_g] = mha.mha_workspace_size(h, 8, 4096, 4096)
        mha.mha_destroy(h)
    st, h = mha.mha_create(1024, 16, mha.MHA_BF16)
    assert mha.mha_workspace_size(h, 8, 4096, 4096) == sizes[16]
    mha.mha_destroy(h)
    # K and V^T shrink by n_g / h: two (B, T, D) fp16 buffers scaled down
    full_kv = 2 * 8 * 4096 * 1024 * 2
    assert sizes[16] - sizes[4] >= full_kv * 3 // 4 - 4096
    assert sizes[4] > sizes[1] > 0
    for dt in (mha.MHA_F32, mha.MHA_BF16):
        st, h = mha.mha_create_grouped(512, 8, 2, dt)
        assert st == mha.MHA_OK
        assert mha.mha_workspace_size(h, 2, 100, 300) > 0
        mha.mha_destroy(h)


def test_decode_validation_without_device_work(mha):
    st, h = mha.mha_create_grouped(1024, 16, 4, mha.MHA_BF16)
    st2, h32 = mha.mha_create(512, 8, mha.MHA_F32)
    fake = 1 << 20
    try:
        ws = mha.mha_decode_workspace_size(h, 4, 2, 128)
        assert ws > 0 and ws % 256 == 0
        assert mha.mha_decode_workspace_size(h, 4, 3, 2) == 0        # T_new > T_max
        assert mha.mha_decode_workspace_size(h, 0, 1, 128) == 0
        assert mha.mha_decode_workspace_size(h32, 4, 1, 128) == 0    # bf16 handles only

        def call(handle=h, **kw):
            args = dict(x=fake, w_qkv=fake, b_qkv=None, w_o=fake, b_o=None, B=4, T_new=2,
                        k_cache=fake, v_cache=fake, T_max=128, cache_len=fake, y=fake,
                        workspace=fake, workspace_bytes=ws, stream=None)
            args.update(kw)
            return mha.mha_decode(handle, *args.values())

        assert call(handle=None) == mha.MHA_ERR_INVALID_ARG
        assert call(k_cache=None) == mha.MHA_ERR_INVALID_ARG
        assert call(cache_len=None) == mha.MHA_ERR_INVALID_ARG
        assert call(cache_len=fake + 2) == mha.MHA_ERR_INVALID_ARG   # misaligned lengths
        assert call(v_cache=fake + 8) == mha.MHA_ERR_INVALID_ARG     # misaligned cache
        assert call(T_new=0) == mha.MHA_ERR_INVALID_ARG
        assert call(T_new=129) == mha.MHA_ERR_INVALID_ARG
        assert call(B=70000) == mha.MHA_ERR_INVALID_ARG
        assert call(workspace_bytes=ws - 1) == mha.MHA_ERR_WORKSPACE
        assert call(handle=h32) == mha.MHA_ERR_UNSUPPORTED
    finally:
        mha.mha_destroy(h)
        mha.mha_destroy(h32)


def test_forward_options_validation(mha):
    st, h = mha.mha_create(512, 8, mha.MHA_BF16)
    st2, h32 = mha.mha_create(512, 8, mha.MHA_F32)
    fake = 1 << 20
    try:
        ws = mha.mha_workspace_size(h, 2, 16, 16)

        def call(opts, handle=h, T=16):
            return mha.mha_forward_ex(handle, fake, None, fake, None, fake, None, 2, T, T, 0,
                                      None, fake, fake, mha.mha_workspace_size(handle, 2, T, T),
                                      opts, None)

        O = mha.mha_forward_options
        assert call(O(2, 0, None, 0)) == mha.MHA_ERR_INVALID_ARG      # residual not 0/1
        assert call(O(0, 3, None, 0)) == mha.MHA_ERR_INVALID_ARG
        assert call(O(0, 0, fake + 4, 0)) == mha.MHA_ERR_INVALID_ARG  # misaligned weights
        assert call(O(0, 1, None, 0), handle=h32) == mha.MHA_ERR_UNSUPPORTED   # bf16 y, fp32 path
        assert call(O(0, 0, fake, 0), T=5000) == mha.MHA_ERR_UNSUPPORTED        # weights, T_k > 4096
        assert call(O(0, 0, None, 0, None, None, fake + 2)) == mha.MHA_ERR_INVALID_ARG  # flag
        assert call(O(0, 0, None, 0, None, None, fake + 2), handle=h32) == mha.MHA_ERR_INVALID_ARG
        assert mha.mha_forward_ex(h, None, None, fake, None, fake, None, 2, 16, 16, 0, None, fake,
                                  fake, ws, O(1, 0, None, 0), None) == mha.MHA_ERR_INVALID_ARG
    finally:
        mha.mha_destroy(h)
        mha.mha_destroy(h32)


def test_noalloc_rejects_before_device_work(mha):
    """mha_forward_noalloc validates like mha_forward and rejects sizes whose
    workspace exceeds the library's scratch, all before touching a device."""
    text = open(HEADER).read()
    m = re.search(r"#define MHA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == mha.MHA_NOALLOC_SCRATCH_BYTES
    st, h = mha.mha_create(1024, 16, mha.MHA_BF16)
    fake = 1 << 20
    try:
        def call(**kw):
            args = dict(x_q=fake, x_kv=None, w_qkv=fake, b_qkv=None, w_o=fake, b_o=None, B=2,
                        T_q=16, T_k=16, causal=0, key_padding_mask=None, y=fake, opts=None,
                        stream=None)
            args.update(kw)
            return mha.mha_forward_noalloc(h, *args.values())
        assert call(x_q=None) == mha.MHA_ERR_INVALID_ARG
        assert call(causal=3) == mha.MHA_ERR_INVALID_ARG
        assert call(y=fake + 4) == mha.MHA_ERR_INVALID_ARG
        # the headline size needs ~272 MiB of workspace
        assert mha.mha_workspace_size(h, 8, 4096, 4096) > mha.MHA_NOALLOC_SCRATCH_BYTES
        assert call(B=8, T_q=4096, T_k=4096, causal=1) == mha.MHA_ERR_WORKSPACE
        # just past the limit, found by bisection on T
        lo, hi = 1, 4096
        while lo + 1 < hi:
            mid = (lo + hi) // 2
            if mha.mha_workspace_size(h, 2, mid, mid) <= mha.MHA_NOALLOC_SCRATCH_BYTES:
                lo = mid
            else:
                hi = mid
        assert call(B=2, T_q=hi, T_k=hi) == mha.MHA_ERR_WORKSPACE
    finally:
        mha.mha_destroy(h)
