"""The C-ABI library loads and exports what include/moe.h declares; host-side
argument checks reject bad calls before anything is launched (no GPU)."""
import ctypes
import os

import pytest

import moe_expert_layer_topk_amd as moe
from gen import slot_layout, CONFIGS


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(moe.LIB_PATH):
        from moe_expert_layer_topk_amd.build import build
        build()
    return moe.lib()


def test_every_declared_symbol_is_exported(L):
    names = moe.declared_symbols()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_strerror(L):
    assert L.moe_abi_version() == 1
    assert L.moe_strerror(0) == b"ok"
    assert L.moe_strerror(-1) == b"invalid argument"


@pytest.mark.parametrize("name", ["C0", "C1", "C3", "C4"])
def test_slot_layout_matches_generator(L, name):
    c = CONFIGS[name]
    for fmt in (0, 1):
        if fmt == 1 and c.I % 128:
            assert moe.slot_bytes(c.H, c.I, fmt) == 0
            continue
        lay = slot_layout(c.H, c.I, fmt)
        assert moe.slot_bytes(c.H, c.I, fmt) == lay["total"][1]
        parts = [k for k in lay if k != "total"]
        for i, p in enumerate(parts):
            assert moe.slot_part_offset(c.H, c.I, fmt, i) == lay[p][0]


def test_slot_bytes_hand_values(L):
    """Slot sizes at hidden 2048, inter 512, worked by hand from the layout:
    FP8 = 2I*H codes + 2I*4 scale + H*I codes + H*4 scale = 2097152 + 4096 +
    1048576 + 8192 = 3158016 (each array already a multiple of 256); int4 =
    I*H + 2I*(H/128)*4 + H*I/2 + H*(I/128)*4 = 1048576 + 65536 + 524288 +
    32768 = 1671168, plus the 16 spare tail bytes rounded up to 256."""
    assert moe.slot_bytes(2048, 512, 0) == 3158016
    assert moe.slot_bytes(2048, 512, 1) == 1671168 + 256
    assert moe.slot_bytes(2048, 768, 0) == 2 * 768 * 2048 + 2 * 768 * 4 + 2048 * 768 + 2048 * 4   # 4732928


def test_align_capacity_formula(L):
    import oracle
    for T, k, E, bm in [(1, 8, 256, 16), (32, 8, 256, 16), (16384, 8, 256, 128), (7, 3, 5, 64), (16, 2, 8, 256)]:
        assert moe.align_capacity(T, k, E, bm) == oracle.align_capacity(T, k, E, bm)


def test_host_checks_reject_bad_arguments(L):
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation
    null = None
    assert L.moe_route(null, null, 4, 8, 2, fake, fake, fake, null) == -1            # no logits
    assert L.moe_route(fake, null, 0, 8, 2, fake, fake, fake, null) == -1            # T = 0
    assert L.moe_route(fake, null, 4, 8, 9, fake, fake, fake, null) == -1            # k > E
    assert L.moe_route(fake, null, 4, 2048, 2, fake, fake, fake, null) == -1         # E > 1024
    assert L.moe_route(fake, null, 4, 64, 33, fake, fake, fake, null) == -1          # k > 32
    assert L.moe_align(fake, 4, 2, 8, 24, fake, fake, fake, fake, fake, fake, fake, null, 0, null) == -1  # block_m
    assert L.moe_align_capacity(4, 2, 8, 7) == -1
    pool = moe.binding.moe_slot_pool(fake, 3158016, 4, fake, 2048, 512)
    bad_h = moe.binding.moe_slot_pool(fake, 3158016, 4, fake, 2000, 512)
    small = moe.binding.moe_slot_pool(fake, 4096, 4, fake, 2048, 512)
    args = (fake, 4, 8, 256, fake, fake, fake, fake)
    assert L.moe_expert_ffn(ctypes.byref(bad_h), *args, 16, 0, fake, fake, 1 << 30, null) == -1
    assert L.moe_expert_ffn(ctypes.byref(small), *args, 16, 0, fake, fake, 1 << 30, null) == -1
    assert L.moe_expert_ffn(ctypes.byref(pool), *args, 128, 0, fake, fake, 1 << 30, null) == -1   # bf16 block_m
    assert L.moe_expert_ffn(ctypes.byref(pool), *args, 16, 1, fake, fake, 1 << 30, null) == -1    # fp8 block_m
    assert L.moe_expert_ffn(ctypes.byref(pool), *args, 16, 7, fake, fake, 1 << 30, null) == -1    # act mode
    assert L.moe_expert_ffn(ctypes.byref(pool), *args, 16, 0, fake, fake, 16, null) == -1         # workspace
    big_t = (fake, 65, 8, 256, fake, fake, fake, fake)
    assert L.moe_expert_ffn(ctypes.byref(pool), *big_t, 16, 0, fake, fake, 1 << 40, null) == -1   # bf16 T > 64
    assert L.moe_dequant_slot(ctypes.byref(pool), 4, fake, fake, null) == -1                     # slot range
    assert L.moe_dequant_slot(ctypes.byref(pool), 0, null, null, null) == -1
    assert L.moe_quant_act(fake, 4, 100, fake, fake, null) == -1                                  # cols % 128
    assert L.moe_quant_act(fake, 0, 256, fake, fake, null) == -1
    assert L.moe_pool_check(ctypes.byref(small), fake, null, null) == -1                          # stride
    assert L.moe_pool_check(ctypes.byref(pool), null, null, null) == -1                           # no err word
    int4_only = moe.binding.moe_slot_pool(fake, moe.slot_bytes(2048, 512, 1), 4, fake, 2048, 512)
    one_short = moe.binding.moe_slot_pool(fake, moe.slot_bytes(2048, 512, 1) - 256, 4, fake, 2048, 512)
    assert L.moe_dequant_slot(ctypes.byref(one_short), 0, fake, fake, null) == -1                 # fits no format
    assert L.moe_dequant_slot(ctypes.byref(int4_only), 4, fake, fake, null) == -1                 # (slot range)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    from moe_expert_layer_topk_amd import binding
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "libmoe.so"))
    with pytest.raises(moe.MoeError):
        binding.lib()
