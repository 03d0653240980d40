"""Host-side checks of libmoe: the library loads without a GPU, exports every
entry point include/moe.h declares, validates configs and computes the
capacity exactly as the oracle does.  No kernel is launched."""
import ctypes
import os
import re

import pytest

import oracle.oracle as O
import sparse_mixture_experts_capacity_amd as moe
from sparse_mixture_experts_capacity_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_symbols():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_header_declares_the_abi():
    names = declared_symbols()
    for must in ("moe_forward", "moe_route", "moe_route_logits", "moe_aux_loss",
                 "moe_workspace_size", "moe_check_config", "moe_last_error",
                 "moe_capacity"):
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert set(declared_symbols()) == set(_lib.EXPORTED_SYMBOLS)


def cfg(**kw):
    base = dict(T=128, d_model=128, d_ff=256, n_experts=8, top_k=2,
                dtype="bf16", capacity_factor=1.25)
    base.update(kw)
    return moe.make_config(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(), moe.MOE_OK),
    (dict(T=0), moe.MOE_OK),
    (dict(T=-1), moe.MOE_EINVAL),
    (dict(top_k=0), moe.MOE_EINVAL),
    (dict(top_k=9), moe.MOE_EINVAL),
    (dict(n_experts=0), moe.MOE_EINVAL),
    (dict(n_experts=257, top_k=2), moe.MOE_EINVAL),
    (dict(n_experts=256, top_k=256), moe.MOE_OK),
    (dict(d_model=0), moe.MOE_EINVAL),
    (dict(d_ff=-64), moe.MOE_EINVAL),
    (dict(n_shared=-1), moe.MOE_EINVAL),
    (dict(gating=2), moe.MOE_EINVAL),
    (dict(dtype=7), moe.MOE_EINVAL),
    (dict(ffn_path=3), moe.MOE_EINVAL),
    (dict(capacity_factor=float("nan")), moe.MOE_EINVAL),
    (dict(capacity_factor=2e6), moe.MOE_EINVAL),
    (dict(out_fp32=2), moe.MOE_EINVAL),
    (dict(T=2 ** 30, top_k=2), moe.MOE_EINVAL),
    (dict(d_model=96), moe.MOE_EUNSUPPORTED),
    (dict(d_ff=100), moe.MOE_EUNSUPPORTED),
    (dict(dtype="f32", d_model=5, d_ff=7), moe.MOE_OK),
    (dict(dtype="f32", ffn_path=moe.PATH_STREAM), moe.MOE_EUNSUPPORTED),
    (dict(overflow=moe.OVERFLOW_REROUTE), moe.MOE_OK),
    (dict(overflow=moe.OVERFLOW_SEQUENTIAL), moe.MOE_OK),
    (dict(overflow=3), moe.MOE_EINVAL),
    (dict(overflow=-1), moe.MOE_EINVAL),
    (dict(weight_layout=moe.WEIGHTS_PACKED), moe.MOE_OK),
    (dict(weight_layout=2), moe.MOE_EINVAL),
    (dict(dtype="f32", weight_layout=moe.WEIGHTS_PACKED), moe.MOE_EUNSUPPORTED),
])
def test_check_config(kw, code):
    c = cfg(**kw)
    if "dtype" in kw and kw["dtype"] == 7:
        c.dtype = 7
    rc = moe.moe_check_config(c)
    assert rc == code, moe.moe_last_error()
    if code != moe.MOE_OK:
        assert moe.moe_last_error()
        assert moe.moe_workspace_size(c) == 0
        assert moe.moe_capacity(c) == -1


def test_null_config():
    assert moe.LIB.moe_check_config(None) == moe.MOE_EINVAL
    assert "NULL" in moe.moe_last_error()


@pytest.mark.parametrize("T,k,E,cf", [
    (2048, 2, 8, 1.25), (16384, 2, 8, 1.0), (16384, 2, 8, 1.5), (100, 2, 2, 1.1),
    (10, 1, 4, 1.0), (1, 1, 8, 1.0), (7, 3, 5, 0.3), (4096, 6, 160, 0.0),
    (333, 2, 7, 1.3333), (64, 2, 8, -1.0), (1000, 8, 64, 2.0 / 3.0),
    (12345, 4, 13, 1e-3), (5, 2, 3, 123456.0), (0, 2, 8, 1.25),
    # tiny positive factors: C is at least 1 (and no exponent overflows)
    (2048, 2, 8, 1e-40), (2048, 2, 8, 1e-60), (2048, 2, 8, 1e-130),
    (2048, 2, 8, 5e-324), (2 ** 30 - 1, 1, 1, 1e-300), (0, 2, 8, 1e-130),
    (2 ** 30 - 1, 1, 256, 999999.999999999), (3, 1, 256, 1.2345678901234567e-7),
])
def test_capacity_matches_oracle(T, k, E, cf):
    c = cfg(T=T, top_k=k, n_experts=E, capacity_factor=cf)
    assert moe.moe_capacity(c) == O.capacity(T, k, E, cf)


def test_workspace_grows_with_tokens():
    sizes = [moe.moe_workspace_size(cfg(T=T)) for T in (1, 64, 1024, 8192)]
    assert all(s > 0 for s in sizes)
    assert sizes == sorted(sizes)
    assert moe.moe_workspace_size(cfg(T=0)) >= 0


def test_struct_layouts_match_the_header():
    # moe_config_t ends with the overflow policy, the weight layout and the
    # fp32-output flag; moe_stats_t with the
    # overflow counters (offsets as the C compiler lays them out on x86-64)
    assert _lib.MoeConfig.overflow.offset == 88 and ctypes.sizeof(_lib.MoeConfig) == 104
    assert _lib.MoeConfig.weight_layout.offset == 92
    assert _lib.MoeConfig.out_fp32.offset == 96
    assert _lib.MoeStats.rounds.offset == 96 and ctypes.sizeof(_lib.MoeStats) == 104


def test_overflow_policies_size_the_workspace():
    # rerouting needs three T*k index arrays; sequential rounds keep every
    # assignment, so the row buffers hold T*k rows instead of E*C
    drop = moe.moe_workspace_size(cfg(T=4096, capacity_factor=1.0))
    rr = moe.moe_workspace_size(cfg(T=4096, capacity_factor=1.0, overflow=moe.OVERFLOW_REROUTE))
    seq = moe.moe_workspace_size(cfg(T=4096, capacity_factor=0.5,
                                     overflow=moe.OVERFLOW_SEQUENTIAL))
    half = moe.moe_workspace_size(cfg(T=4096, capacity_factor=0.5))
    assert rr >= drop + 3 * 4 * 4096 * 2
    assert seq > half
    # the reported capacity is the policy-independent C
    for pol in (moe.OVERFLOW_DROP, moe.OVERFLOW_REROUTE, moe.OVERFLOW_SEQUENTIAL):
        assert moe.moe_capacity(cfg(T=4096, capacity_factor=0.5, overflow=pol)) == 512


def test_router_backward_argument_checks():
    # host-side validation only: nothing is launched
    c = cfg(T=64)
    assert moe.LIB.moe_router_backward(None, None, None, 0.0, 0.0, ctypes.byref(c), None, None,
                                       None, None) == moe.MOE_EINVAL
    assert "dout" in moe.moe_last_error()
    fake = 256   # never dereferenced: the checks fail first
    assert moe.LIB.moe_router_backward(None, None, fake, 0.0, 0.0, ctypes.byref(c), fake, fake,
                                       None, None) == moe.MOE_EINVAL
    assert "x must be" in moe.moe_last_error()
    assert moe.LIB.moe_router_backward(None, None, fake, float("inf"), 0.0, ctypes.byref(c), fake,
                                       None, None, None) == moe.MOE_EINVAL
    assert moe.LIB.moe_router_backward(None, None, fake, 0.0, float("nan"), ctypes.byref(c),
                                       fake, None, None, None) == moe.MOE_EINVAL
    assert moe.LIB.moe_router_backward(None, None, fake, 0.0, 0.0, ctypes.byref(c), fake, None,
                                       None, None) == moe.MOE_EWORKSPACE
    assert moe.LIB.moe_router_backward(None, None, None, 0.0, 0.0, ctypes.byref(cfg(T=0)), None,
                                       None, None, None) == moe.MOE_OK


def test_misaligned_tensors_are_refused():
    # host-side validation only: nothing is launched.  The kernels move x,
    # W_gate, the expert weights and out in 16-byte pieces, so a pointer 2
    # bytes into an allocation (a bf16 view starting one element in) is an
    # argument error, reported before the workspace is looked at.
    c = cfg(T=64)
    ok, off = 256, 258
    for args in ([off, ok, ok, ok, ok, ok], [ok, off, ok, ok, ok, ok], [ok, ok, off, ok, ok, ok],
                 [ok, ok, ok, off, ok, ok], [ok, ok, ok, ok, off, ok], [ok, ok, ok, ok, ok, off]):
        x, wg, w1, w3, w2, out = args
        rc = moe.LIB.moe_forward(x, wg, w1, w3, w2, ctypes.byref(c), out, None)
        assert rc == moe.MOE_EINVAL
        assert "16-byte aligned" in moe.moe_last_error()
    idx = 512
    assert moe.LIB.moe_route(off, ok, ctypes.byref(c), None, idx, None, None, None, None, None,
                             None) == moe.MOE_EINVAL
    assert "16-byte aligned" in moe.moe_last_error()
    assert moe.LIB.moe_router_backward(off, ok, ok, 0.0, 0.0, ctypes.byref(c), ok, ok, None,
                                       None) == moe.MOE_EINVAL
    assert "16-byte aligned" in moe.moe_last_error()
    assert moe.LIB.moe_pack_weights(ok, ok, ok, ctypes.byref(cfg()), ok, off,
                                    ok) == moe.MOE_EINVAL
    assert "16-byte aligned" in moe.moe_last_error()
    # aligned pointers get past the check to the missing workspace
    assert moe.LIB.moe_forward(ok, ok, ok, ok, ok, ctypes.byref(c), ok, None) == moe.MOE_EWORKSPACE
    # no tokens: nothing is read, so nothing is checked
    assert moe.LIB.moe_forward(off, off, off, off, off, ctypes.byref(cfg(T=0)), off,
                               None) == moe.MOE_OK


@pytest.mark.parametrize("d,F,E,S", [(128, 256, 8, 0), (192, 320, 4, 2), (4096, 14336, 8, 0),
                                     (5120, 1536, 160, 2)])
def test_packed_weight_sizes(d, F, E, S):
    # W1/W3 rows padded to a multiple of 128 columns, W2 rows to 256
    c = cfg(d_model=d, d_ff=F, n_experts=E, n_shared=S)
    w13, w2 = moe.moe_packed_weight_bytes(c)
    pad = lambda v, m: -(-v // m) * m
    assert w13 == 2 * (E + S) * d * pad(F, 128)
    assert w2 == 2 * (E + S) * F * pad(d, 256)
    assert w13 >= 2 * (E + S) * d * F and w2 >= 2 * (E + S) * F * d


def test_pack_weights_argument_checks():
    # host-side validation only: nothing is launched
    c = cfg()
    with pytest.raises(moe.MoeError) as e:
        moe.moe_pack_weights(None, None, None, c, None, None, None)
    assert e.value.code == moe.MOE_EINVAL
    with pytest.raises(moe.MoeError) as e:
        moe.moe_packed_weight_bytes(cfg(dtype="f32"))
    assert e.value.code == moe.MOE_EUNSUPPORTED
    fake = 256   # never dereferenced: the checks fail first
    assert moe.LIB.moe_pack_weights(fake, fake, fake, ctypes.byref(cfg(dtype="f32")), fake, fake,
                                    fake) == moe.MOE_EUNSUPPORTED


def test_missing_library_fails_loudly(tmp_path):
    # no fallback: a copy of the package without libmoe.so refuses to import
    import shutil
    import subprocess
    import sys
    pkg = os.path.join(ROOT, "sparse_mixture_experts_capacity_amd")
    dst = tmp_path / "sparse_mixture_experts_capacity_amd"
    dst.mkdir()
    for f in os.listdir(pkg):
        if f.endswith(".py"):
            shutil.copy(os.path.join(pkg, f), dst / f)
    r = subprocess.run([sys.executable, "-c", "import sparse_mixture_experts_capacity_amd"],
                       cwd=str(tmp_path), capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "libmoe.so is missing" in r.stderr


def test_noalloc_refuses_layers_beyond_its_scratch():
    # checked before the scratch array is looked up, so no GPU is touched:
    # the Mixtral-shaped prefill layer needs far more than the 64 MiB
    big = cfg(T=2048, d_model=4096, d_ff=14336, n_experts=8, top_k=2)
    assert moe.moe_workspace_size(big) > 64 << 20
    fake = 256   # never dereferenced: the size check fails first
    rc = moe.LIB.moe_forward_noalloc(fake, fake, fake, fake, fake, ctypes.byref(big), fake, None)
    assert rc == moe.MOE_EWORKSPACE
    assert "moe_forward_noalloc holds 67108864" in moe.moe_last_error()
    # invalid configurations are refused as by moe_forward
    bad = cfg(top_k=0)
    assert moe.LIB.moe_forward_noalloc(fake, fake, fake, fake, fake, ctypes.byref(bad), fake,
                                       None) == moe.MOE_EINVAL


def test_debug_canaries_grow_the_workspace():
    c = cfg(T=512)
    plain = moe.moe_workspace_size(c)
    moe.moe_debug_canaries(True)
    try:
        guarded = moe.moe_workspace_size(c)
    finally:
        moe.moe_debug_canaries(False)
    assert guarded > plain
    assert (guarded - plain) % 256 == 0 and (guarded - plain) // 256 >= 20
    assert moe.moe_workspace_size(c) == plain
