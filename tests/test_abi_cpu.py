"""The C-ABI library loads on a machine without a GPU and exports every
symbol include/moe.h declares; host-only helpers answer correctly. No compute
call is made here."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names += re.findall(r"^[A-Za-z_][\w \*]*?\b(moe_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def libmoe():
    import quantized_moe_expert_sigmoid_amd as m
    if not os.path.exists(m.LIB_PATH):
        from quantized_moe_expert_sigmoid_amd import build
        build.build(force=False)
    return m.lib()


def test_header_declares_the_abi():
    names = declared_functions()
    for n in ("moe_router_topk", "moe_expert_ffn_q4", "moe_expert_ffn_q8", "moe_expert_ffn_q2", "moe_combine",
              "moe_quantize_rows", "moe_quantize_act_i8", "moe_bucket_tokens", "moe_ctx_create"):
        assert n in names


def test_every_declared_symbol_is_exported(libmoe):
    missing = [n for n in declared_functions() if not hasattr(libmoe, n)]
    assert not missing, missing


def test_binding_covers_the_header():
    import quantized_moe_expert_sigmoid_amd as m
    assert set(declared_functions()) == set(m.exported_names())


def test_host_helpers(libmoe):
    import quantized_moe_expert_sigmoid_amd as m
    assert libmoe.moe_abi_version() == 2
    n, offs = m.moe_expert_block_layout(4, 6144, 2048)
    assert n == 18_915_328 and offs[0] == 0 and offs[1] == 6_291_456 and offs[5] == 18_915_328 - 4 * 6144
    assert m.moe_expert_block_layout(2, 6144, 2048)[0] == 9_478_144
    assert m.moe_expert_block_layout(8, 6144, 2048)[0] == 37_789_696
    with pytest.raises(m.MoeError):
        m.moe_expert_block_layout(3, 6144, 2048)
