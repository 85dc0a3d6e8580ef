"""The C ABI library on the CPU: it loads, exports every entry point the header
declares, sizes workspaces, and rejects bad arguments before any HIP call."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mi355x.h")
LIB = os.path.join(ROOT, "sigmoid_top_routing_router_amd", "libmoe_mi355x.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    from sigmoid_top_routing_router_amd import _lib
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert "moe_forward" in names and "moe_route" in names and "moe_eqb_bias" in names
    for n in names:
        assert hasattr(lib, n), n
    from sigmoid_top_routing_router_amd import _lib
    assert sorted(_lib.EXPORTED) == names


def test_abi_version_and_status_strings(lib):
    assert lib.moe_abi_version() == 2
    assert lib.moe_status_string(0) == b"MOE_OK"
    assert lib.moe_status_string(3) == b"MOE_ERR_WORKSPACE_TOO_SMALL"


def test_struct_layouts_match_header(tmp_path):
    """ctypes mirrors of the header's structs agree with the C compiler."""
    import shutil
    import subprocess
    from sigmoid_top_routing_router_amd._lib import MoeAux, MoeFp8Weights, MoeProblem, MoeWeights
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    prog = tmp_path / "layout.c"
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', 'int main(void){']
    for st, cls in (("moe_problem_t", MoeProblem), ("moe_weights_t", MoeWeights),
                    ("moe_aux_t", MoeAux), ("moe_fp8_weights_t", MoeFp8Weights)):
        lines.append(f'printf("{st} %zu\\n", sizeof({st}));')
        for f, _ in cls._fields_:
            lines.append(f'printf("{st}.{f} %zu\\n", offsetof({st}, {f}));')
    lines.append('return 0;}')
    prog.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run([cc, str(prog), "-o", str(exe)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                  check=True).stdout.splitlines())
    for st, cls in (("moe_problem_t", MoeProblem), ("moe_weights_t", MoeWeights),
                    ("moe_aux_t", MoeAux), ("moe_fp8_weights_t", MoeFp8Weights)):
        assert int(got[st]) == C.sizeof(cls), st
        for f, _ in cls._fields_:
            assert int(got[f"{st}.{f}"]) == getattr(cls, f).offset, (st, f)


def _problem(**kw):
    from sigmoid_top_routing_router_amd._lib import MoeProblem
    base = dict(N=16384, d=2560, E=384, K=6, h=512, n_shared=1, h_shared=512, flags=1,
                logit_offset=None, logits_in=None)
    base.update(kw)
    return MoeProblem(**base)


def test_forward_workspace_sizes(lib):
    p = _problem()
    b = lib.moe_forward_workspace_bytes(C.byref(p))
    pairs = 16384 * 6
    # at least H and the per-pair expert outputs in bf16 plus the logits
    assert b >= pairs * (512 + 2560) * 2 + 16384 * 384 * 4
    assert b < 2 * (pairs * (512 + 2560) * 2 + 16384 * 384 * 4 + 16384 * (512 + 2560) * 2)
    for bad in (dict(K=0), dict(K=9), dict(E=6), dict(E=385), dict(d=100), dict(h=48),
                dict(n_shared=2), dict(N=0), dict(flags=16)):
        assert lib.moe_forward_workspace_bytes(C.byref(_problem(**bad))) == 0, bad


def test_eqb_workspace_sizes(lib):
    b16 = lib.moe_eqb_workspace_bytes(65536, 384, 16)
    b32 = lib.moe_eqb_workspace_bytes(65536, 384, 32)
    assert b16 >= 2 * 384 * 256 * 4 and b32 >= 4 * 384 * 256 * 4 and b32 > b16
    assert lib.moe_eqb_workspace_bytes(65536, 384, 8) == 0


@pytest.mark.parametrize("N,E,K,status", [(0, 384, 6, 2), (10, 384, 0, 2), (10, 384, 9, 2),
                                          (10, 6, 6, 2), (10, 385, 6, 2)])
def test_route_rejects_shapes_without_gpu(lib, N, E, K, status):
    buf = C.create_string_buffer(64)
    p = C.cast(buf, C.c_void_p)
    assert lib.moe_route(p, None, N, E, K, p, p, None, None, None) == status
    assert lib.moe_last_error_message() != b""


def test_route_rejects_null_and_misaligned(lib):
    buf = C.create_string_buffer(64)
    p = C.cast(buf, C.c_void_p).value
    assert lib.moe_route(None, None, 4, 8, 2, p, p, None, None, None) == 1
    assert lib.moe_route(p + 1, None, 4, 8, 2, p, p, None, None, None) == 1


def test_eqb_rejects_bad_arguments(lib):
    buf = C.create_string_buffer(1024)
    p = C.cast(buf, C.c_void_p).value
    assert lib.moe_eqb_bias(p, None, None, 4, 8, 2, 12, p, None, p, 1 << 20, None) == 1
    # too small workspace
    assert lib.moe_eqb_bias(p, None, None, 4, 8, 2, 16, p, None, p & ~255 or p, 16, None) in (1, 3)


def test_forward_rejects_bad_arguments(lib):
    from sigmoid_top_routing_router_amd._lib import MoeWeights
    buf = C.create_string_buffer(4096)
    p16 = (C.cast(buf, C.c_void_p).value + 15) // 16 * 16
    w = MoeWeights(p16, p16, p16, p16, p16, p16, p16)
    prob = _problem(N=4, d=64, E=4, K=2, h=32, h_shared=32)
    # NULL x
    assert lib.moe_forward(C.byref(prob), C.byref(w), None, None, p16, None, p16, 1 << 30, None) == 1
    # misaligned weights
    w2 = MoeWeights(p16 + 2, p16, p16, p16, p16, p16, p16)
    assert lib.moe_forward(C.byref(prob), C.byref(w2), p16, None, p16, None, p16, 1 << 30, None) == 1
    # offset together with logits_in
    prob2 = _problem(N=4, d=64, E=4, K=2, h=32, h_shared=32, logit_offset=p16, logits_in=p16)
    assert lib.moe_forward(C.byref(prob2), C.byref(w), p16, None, p16, None, p16, 1 << 30, None) == 1
    # workspace too small (no HIP call made: the check comes first)
    ws = (p16 + 255) // 256 * 256
    assert lib.moe_forward(C.byref(prob), C.byref(w), p16, None, p16, None, ws, 64, None) == 3
    # unsupported shape
    prob3 = _problem(N=4, d=96, E=4, K=2, h=32, h_shared=32)
    assert lib.moe_forward(C.byref(prob3), C.byref(w), p16, None, p16, None, ws, 1 << 30, None) == 2


def test_eqb_state_sizes(lib):
    s16 = lib.moe_eqb_state_bytes(384, 16)
    s32 = lib.moe_eqb_state_bytes(384, 32)
    assert s16 >= 2 * 384 * 256 * 4 and s32 >= 4 * 384 * 256 * 4 and s32 > s16
    for E, kb in ((1, 16), (385, 16), (384, 8)):
        assert lib.moe_eqb_state_bytes(E, kb) == 0


def test_eqb_parts_reject_bad_arguments(lib):
    """Every check comes before any HIP call: these run without a GPU."""
    buf = C.create_string_buffer(1 << 20)
    base = C.cast(buf, C.c_void_p).value
    st = (base + 255) // 256 * 256
    need = lib.moe_eqb_state_bytes(8, 16)
    # begin: bad key_bits, misaligned state, too small state, bad E
    assert lib.moe_eqb_begin(8, 12, st, need, None) == 1
    assert lib.moe_eqb_begin(8, 16, st + 4, need, None) == 1
    assert lib.moe_eqb_begin(8, 16, st, need - 1, None) == 3
    assert lib.moe_eqb_begin(400, 16, st, 1 << 19, None) == 2
    # accumulate: pass out of range, NULL alpha, bad N
    assert lib.moe_eqb_accumulate(2, st, st, 4, 8, 16, st, need, None) == 1
    assert lib.moe_eqb_accumulate(-1, st, st, 4, 8, 16, st, need, None) == 1
    assert lib.moe_eqb_accumulate(0, st, None, 4, 8, 16, st, need, None) == 1
    assert lib.moe_eqb_accumulate(0, st, st, 0, 8, 16, st, need, None) == 2
    # select: beta_out required at the last pass; K and E checked
    assert lib.moe_eqb_select(1, 4, 8, 2, 16, None, None, st, need, None) == 1
    need32 = lib.moe_eqb_state_bytes(8, 32)
    assert lib.moe_eqb_select(4, 4, 8, 2, 32, st, None, st, need32, None) == 1
    assert lib.moe_eqb_select(3, 4, 8, 2, 32, st, None, st, need, None) == 3
    assert lib.moe_eqb_select(0, 4, 8, 8, 16, st, None, st, need, None) == 2
    assert lib.moe_last_error_message() != b""


def test_forward_rejects_operands_over_four_gib(lib):
    # x [N, d] in bf16 at or above 4 GiB: N * 8192 * 2 >= 2^32
    assert lib.moe_forward_workspace_bytes(C.byref(_problem(N=1 << 18, d=8192))) == 0
    # the routed hidden rows [N*K, h]: 2^20 * 8 * 512 * 2 = 8 GiB
    assert lib.moe_forward_workspace_bytes(C.byref(_problem(N=1 << 20, d=64, K=8))) == 0
    # just below the limits is accepted
    assert lib.moe_forward_workspace_bytes(C.byref(_problem(N=1 << 17, d=8192, K=2))) > 0


def test_route_stats_rejects_bad_arguments(lib):
    buf = C.create_string_buffer(4096)
    p = (C.cast(buf, C.c_void_p).value + 15) // 16 * 16
    assert lib.moe_route_stats(None, None, None, 4, 8, 2, 1e-3, p, p, None) == 1
    assert lib.moe_route_stats(p, None, None, 4, 8, 2, 1e-3, None, p, None) == 1
    assert lib.moe_route_stats(p, None, None, 4, 8, 2, 1e-3, p, p + 4, None) == 1
    assert lib.moe_route_stats(p, p + 2, None, 4, 8, 2, 1e-3, p, p, None) == 1
    assert lib.moe_route_stats(p, None, None, 4, 8, 9, 1e-3, p, p, None) == 2
    assert lib.moe_route_stats(p, None, None, 0, 8, 2, 1e-3, p, p, None) == 2


def test_route_stats_struct_matches_header(tmp_path):
    import subprocess
    from sigmoid_top_routing_router_amd._lib import MoeRouteStats
    src = tmp_path / "s.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "moe_mi355x.h"\n'
                   'int main(void){printf("%zu %zu %zu %zu\\n", sizeof(moe_route_stats_t),'
                   ' offsetof(moe_route_stats_t, overlap), offsetof(moe_route_stats_t, near_ties),'
                   ' offsetof(moe_route_stats_t, min_load));return 0;}\n')
    exe = tmp_path / "s"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    assert got == [C.sizeof(MoeRouteStats), MoeRouteStats.overlap.offset,
                   MoeRouteStats.near_ties.offset, MoeRouteStats.min_load.offset]


def test_lei_rejects_bad_arguments(lib):
    buf = C.create_string_buffer(1 << 16)
    base = C.cast(buf, C.c_void_p).value
    p = (base + 255) // 256 * 256
    need = lib.moe_lei_workspace_bytes(8)
    assert need >= 8 * 8 and lib.moe_lei_workspace_bytes(1) == 0
    args = dict(logits=p, ids=p, g=None, N=4, E=8, K=2, lam=1e-5, tau=1.0, gout=p + 1024,
                dz=p + 2048, inj=None, ws=p + 4096, wsb=need)

    def call(**kw):
        a = dict(args, **kw)
        return lib.moe_lei_backward(a["logits"], a["ids"], a["g"], a["N"], a["E"], a["K"],
                                    a["lam"], a["tau"], a["gout"], a["dz"], a["inj"], a["ws"],
                                    a["wsb"], None)
    assert call(ids=None) == 1
    assert call(gout=None, dz=None) == 1
    assert call(logits=None) == 1            # grad_logits needs the logits
    assert call(tau=0.0) == 1
    assert call(tau=float("nan")) == 1
    assert call(lam=float("inf")) == 1
    assert call(dz=p) == 1                   # aliases the logits
    assert call(ws=p + 4100) == 1            # misaligned workspace
    assert call(wsb=need - 1) == 3
    assert call(K=9) == 2


def test_stage_timing_modes(lib):
    assert lib.moe_stage_timing(3) == 1 and lib.moe_stage_timing(-1) == 1
    assert lib.moe_stage_timing(2) == 0 and lib.moe_stage_timing(0) == 0


def test_fp8_workspace_sizes(lib):
    p = _problem()
    b8 = lib.moe_forward_fp8_workspace_bytes(C.byref(p))
    b16 = lib.moe_forward_workspace_bytes(C.byref(p))
    pairs = 16384 * 6
    # E4M3 x and H plus bf16 per-pair outputs: between the codes and the bf16 sizes
    assert pairs * (512 + 2560 * 2) < b8 < b16
    for bad in (dict(d=192), dict(h=96), dict(h_shared=64), dict(d=100)):
        assert lib.moe_forward_fp8_workspace_bytes(C.byref(_problem(**bad))) == 0, bad
    # h_shared is free when there is no shared expert
    assert lib.moe_forward_fp8_workspace_bytes(C.byref(_problem(n_shared=0, h_shared=64))) > 0


def test_fp8_entry_points_reject_bad_arguments(lib):
    from sigmoid_top_routing_router_amd._lib import MoeFp8Weights
    buf = C.create_string_buffer(4096)
    p16 = (C.cast(buf, C.c_void_p).value + 255) // 256 * 256
    full = [p16] * 13
    prob = _problem(N=4, d=128, E=4, K=2, h=128, h_shared=128)
    w = MoeFp8Weights(*full)
    # NULL block scales of the routed gate
    w_nos = MoeFp8Weights(*(full[:2] + [None] + full[3:]))
    assert lib.moe_forward_fp8(C.byref(prob), C.byref(w_nos), p16, None, p16, None, p16,
                               1 << 30, None) == 1
    # misaligned codes
    w_mis = MoeFp8Weights(*(full[:1] + [p16 + 8] + full[2:]))
    assert lib.moe_forward_fp8(C.byref(prob), C.byref(w_mis), p16, None, p16, None, p16,
                               1 << 30, None) == 1
    # widths that are not multiples of 128
    prob_d = _problem(N=4, d=64, E=4, K=2, h=128, h_shared=128)
    assert lib.moe_forward_fp8(C.byref(prob_d), C.byref(w), p16, None, p16, None, p16,
                               1 << 30, None) == 2
    # workspace too small
    assert lib.moe_forward_fp8(C.byref(prob), C.byref(w), p16, None, p16, None, p16, 64,
                               None) == 3
    # quantisers: shapes checked first, empty inputs enqueue nothing
    assert lib.moe_fp8_quantize_rows(p16, 4, 100, p16, p16, None) == 2
    assert lib.moe_fp8_quantize_rows(p16, -1, 128, p16, p16, None) == 2
    assert lib.moe_fp8_quantize_rows(p16 + 2, 4, 128, p16, p16, None) == 1
    assert lib.moe_fp8_quantize_rows(None, 0, 128, None, None, None) == 0
    assert lib.moe_fp8_quantize_blocks(p16, -1, 128, 128, p16, p16, None) == 2
    assert lib.moe_fp8_quantize_blocks(p16, 1, 0, 128, p16, p16, None) == 2
    assert lib.moe_fp8_quantize_blocks(p16, 1, 128, 128, p16, None, None) == 1
    assert lib.moe_fp8_quantize_blocks(None, 0, 128, 128, None, None, None) == 0


def test_pack_gateup_arguments_and_flag(lib):
    buf = C.create_string_buffer(8192)
    p16 = (C.cast(buf, C.c_void_p).value + 15) // 16 * 16
    f = lib.moe_pack_gateup_weights
    assert f(p16, -1, 32, 64, p16 + 4096, None) == 2    # count below 0
    assert f(p16, 1, 32, 100, p16 + 4096, None) == 2    # cols not a multiple of 64
    assert f(p16, 1, 0, 64, p16 + 4096, None) == 2      # no rows
    assert f(None, 1, 8, 64, p16 + 4096, None) == 1     # NULL input
    assert f(p16 + 8, 1, 8, 64, p16 + 4096, None) == 1  # misaligned input
    assert f(p16, 1, 8, 64, p16 + 512, None) == 1       # output overlaps the 1 KiB input
    assert f(None, 0, 8, 64, None, None) == 0            # empty: nothing to enqueue
    # MOE_PACKED_GATEUP: accepted with bf16 and with E4M3 experts
    assert lib.moe_forward_workspace_bytes(C.byref(_problem(flags=4))) > 0
    assert lib.moe_forward_fp8_workspace_bytes(C.byref(_problem(flags=5))) > 0
