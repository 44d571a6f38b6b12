"""The C-ABI library loads on the CPU and exports every symbol its header
declares; the binding's option struct matches the header's layout.  No compute
call is made here."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tsg.h")
LIB = os.path.join(ROOT, "tile_level_communication_signaled_amd", "libtsg.so")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:tsg_status|void|const char\*|size_t)\s+\**(\w+)\s*\(", txt, flags=re.M)))


def test_header_declares_the_four_paths():
    names = _declared()
    for n in ("gemm_ag_overlap", "gemm_rs_overlap", "mlp2_pipelined", "moe_expert_combine",
              "tsg_ctx_create", "tsg_ctx_destroy", "tsg_check", "tsg_workspace_bytes"):
        assert n in names


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    for n in _declared():
        assert re.search(rf"\bT {n}$", out, flags=re.M), n


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_binding_exports_match_header():
    import tile_level_communication_signaled_amd as tsg
    assert sorted(tsg.EXPORTS) == _declared()


def test_opts_struct_layout_matches_header(tmp_path):
    src = tmp_path / "sz.c"
    src.write_text('#include "tsg.h"\n#include <stdio.h>\n#include <stddef.h>\n'
                   'int main(void){printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(tsg_opts), '
                   'offsetof(tsg_opts, timeout_ms), offsetof(tsg_opts, timeline), offsetof(tsg_opts, comm_tile), '
                   'offsetof(tsg_opts, pull_units), offsetof(tsg_opts, stage_dtype), '
                   'offsetof(tsg_opts, arrival_gbps), offsetof(tsg_opts, copy_engine), '
                   'offsetof(tsg_opts, channels), offsetof(tsg_opts, ep_ranks), offsetof(tsg_opts, ep_rank));'
                   'return 0;}\n')
    exe = tmp_path / "sz"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()
    sys.path.insert(0, ROOT)
    if not os.path.exists(LIB):
        pytest.skip("library not built")
    import tile_level_communication_signaled_amd as tsg
    assert [int(v) for v in got] == [ctypes.sizeof(tsg.Opts), tsg.Opts.timeout_ms.offset, tsg.Opts.timeline.offset,
                                      tsg.Opts.comm_tile.offset, tsg.Opts.pull_units.offset,
                                      tsg.Opts.stage_dtype.offset, tsg.Opts.arrival_gbps.offset,
                                      tsg.Opts.copy_engine.offset, tsg.Opts.channels.offset,
                                      tsg.Opts.ep_ranks.offset, tsg.Opts.ep_rank.offset]


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_workspace_query_is_host_only():
    import tile_level_communication_signaled_amd as tsg
    assert tsg.workspace_bytes(tsg.OP_AG, [1, 1, 1, 1, 1]) == 0


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_moe_workspace_layout_is_consistent():
    # host-only query: regions in order, 256-byte aligned, each large enough
    # for what the header says it holds, and the total equal to the size query
    import tile_level_communication_signaled_amd as tsg
    T, H, I, E, k = 4096, 4096, 1408, 8, 2
    L = tsg.moe_workspace_layout([T, H, I, E, k])
    assert L["total"] == tsg.workspace_bytes(tsg.OP_MOE, [T, H, I, E, k])
    assert L["rows_max"] == L["rb_max"] * L["bm"]
    assert L["rows_max"] >= T * k + E * (L["bm"] - 1)
    sizes = {"meta": 8, "offs": 4 * (E + 1), "poffs": 4 * (E + 1), "rb_expert": 4 * L["rb_max"],
             "row_pair": 4 * L["rows_max"], "row_token": 4 * L["rows_max"], "pair_row": 4 * T * k,
             "rb_mask": 4 * L["rb_max"], "rb_order": 4 * L["rb_max"], "h": 2 * L["rows_max"] * I,
             "y": 4 * L["rows_max"] * H}
    order = ["meta", "offs", "poffs", "rb_expert", "row_pair", "row_token", "pair_row", "rb_mask", "rb_order", "h",
             "y"]
    for a, b in zip(order, order[1:] + ["total"]):
        assert L[a] % 256 == 0 and L[a] + sizes[a] <= L[b], (a, b)
    with pytest.raises(tsg.TsgError):
        tsg.moe_workspace_layout([T, H, I, E, 3])
