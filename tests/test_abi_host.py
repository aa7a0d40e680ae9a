"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every entry point the header declares, computes sizes in closed form, and
rejects bad arguments before making any HIP call."""
import ctypes
import os
import re

import pytest

from mixture_experts_routed_amd import abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_routed.h")


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^(?:int|const char \*)\s*\**\s*(moe_\w+)\s*\(", txt, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("moe_plan", "moe_gather", "moe_expert_ffn", "moe_combine", "moe_forward"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = abi.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    assert set(declared_functions()) == set(abi.EXPORTS)


def test_plan_sizes_closed_form():
    z = abi.moe_plan_sizes(2048, 10, 512, 16)
    assert (z.nent, z.nblk) == (20480, 20)
    # ceil((20480 + 512*15) / 16) * 16
    assert z.max_rows == (20480 + 512 * 15 + 15) // 16 * 16 == 28160
    assert z.max_tiles == 28160 // 16
    assert z.scratch_bytes == 20 * 514 * 4
    z = abi.moe_plan_sizes(4, 8, 128, 16)  # fewer entries than experts
    assert z.max_rows == (32 + 32 * 15 + 15) // 16 * 16 == 512


def test_status_strings():
    assert abi.moe_status_str(0) == "ok"
    assert abi.moe_status_str(1) == "invalid argument"
    assert abi.moe_status_str(99) == "unknown status"


@pytest.mark.parametrize("T,K,E,tm,rc", [
    (0, 1, 8, 16, 1), (4, 0, 8, 16, 1), (4, 2, 0, 16, 1), (4, 2, 8, 0, 1),
    (4, 2, 1025, 16, 2), (2 ** 30, 4, 8, 16, 1),
])
def test_plan_sizes_errors(T, K, E, tm, rc):
    z = abi.PlanSizes()
    assert abi.lib().moe_plan_sizes(T, K, E, tm, ctypes.byref(z)) == rc


# fake, well-aligned addresses: every call below must return before touching them
A = 1 << 20


def test_plan_rejects_null_misaligned_and_small_scratch():
    L = abi.lib()
    ok = [A] * 10
    assert L.moe_plan(None, A, 4, 2, 8, 16, *ok[:8], A, 4096, None) == 1          # NULL ids
    assert L.moe_plan(A + 2, A, 4, 2, 8, 16, *ok[:8], A, 4096, None) == 1         # misaligned
    assert L.moe_plan(A, A, 4, 2, 8, 16, *ok[:8], A, 7, None) == 1                # small scratch
    assert L.moe_plan(A, A, 4, 2, 2000, 16, *ok[:8], A, 1 << 20, None) == 2       # E too large


def test_gather_combine_ffn_forward_reject_bad_arguments():
    L = abi.lib()
    assert L.moe_gather(A, 5, 4, 64, A, A, 64, A, None) == 1        # bad dtype
    assert L.moe_gather(A, 1, 4, 60, A, A, 64, A, None) == 1        # d % 8
    assert L.moe_gather(A + 8, 1, 4, 64, A, A, 64, A, None) == 1    # x not 16-byte aligned
    assert L.moe_combine(A, 64, A, 4, 2, 12, A, None) == 1          # d % 8
    assert L.moe_combine(A, 64, A, 0, 2, 16, A, None) == 1          # T < 1
    assert L.moe_combine(A + 4, 64, A, 4, 2, 16, A, None) == 1      # y misaligned
    need = ctypes.c_size_t()
    assert L.moe_ffn_scratch_bytes(8, 64, 128, 16, 256, 1, ctypes.byref(need)) == 0
    args = [A, A, A, A, 1, 8, 64, 128, 16, A, A, A, A, 256, A, A, A]
    assert L.moe_expert_ffn(*args, need.value - 1, None) == 1       # small scratch
    bad = list(args)
    bad[7] = 100                                                     # f % 8
    assert L.moe_expert_ffn(*bad, need.value, None) == 1
    bad = list(args)
    bad[5] = 4096                                                    # E too large
    assert L.moe_expert_ffn(*bad, 1 << 30, None) == 2
    ws = ctypes.c_size_t()
    assert L.moe_forward_workspace(64, 2, 8, 128, 256, 16, 0, ctypes.byref(ws)) == 0
    fargs = [A, A, A, A, A, A, 0, 64, 2, 8, 128, 256, 16, A]
    assert L.moe_forward(*fargs, ws.value - 1, A, None) == 1        # small workspace
    assert L.moe_forward(A, A, A, A, A, A, 0, 64, 2, 8, 128, 256, 16, A + 128, ws.value, A,
                         None) == 1                                   # workspace not 256-aligned


def test_packed_weight_sizes_and_rejects():
    L = abi.lib()
    v = ctypes.c_size_t()
    # prefill shape: no padding (f = 768 = 3 x 256 columns, d = 2560 = 80 x 32 K)
    assert L.moe_packed_weight_bytes(512, 2560, 768, 1, 0, ctypes.byref(v)) == 0
    assert v.value == 512 * 2560 * 768 * 2
    assert L.moe_packed_weight_bytes(512, 2560, 768, 1, 1, ctypes.byref(v)) == 0
    assert v.value == 512 * 2560 * 768 * 2
    # ragged: columns padded to 256 (gate/up) / 512 (down), K to 32 (16-bit) / 16 (fp32)
    assert L.moe_packed_weight_bytes(3, 328, 200, 1, 0, ctypes.byref(v)) == 0
    assert v.value == 3 * 256 * 352 * 2
    assert L.moe_packed_weight_bytes(3, 328, 200, 0, 1, ctypes.byref(v)) == 0
    assert v.value == 3 * 512 * 208 * 4
    assert L.moe_packed_weight_bytes(3, 328, 200, 1, 2, ctypes.byref(v)) == 1   # bad kind
    assert L.moe_packed_weight_bytes(3, 330, 200, 1, 0, ctypes.byref(v)) == 1   # d % 8
    assert L.moe_packed_weight_bytes(2000, 64, 64, 1, 0, ctypes.byref(v)) == 2  # E too large
    assert L.moe_pack_weights(A, 1, 3, 328, 200, 0, A, 10, None) == 1          # small output
    assert L.moe_pack_weights(A + 8, 1, 3, 328, 200, 0, A, 1 << 30, None) == 1  # misaligned


def test_forward_layout_is_consistent():
    L = abi.moe_forward_layout(2048, 10, 512, 2560, 768, 16, abi.MOE_F16)
    z = abi.moe_plan_sizes(2048, 10, 512, 16)
    offs = [L.cnt, L.eoff, L.tiles, L.stok, L.sw, L.pos, L.boff, L.meta, L.plan_scratch, L.xs, L.h,
            L.y, L.ffn_scratch, L.total]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert L.h - L.xs >= z.max_rows * 2560 * 2
    assert L.y - L.h >= z.max_rows * 768 * 2
    assert L.ffn_scratch - L.y >= z.max_rows * 2560 * 4
    assert abi.moe_forward_workspace(2048, 10, 512, 2560, 768, 16, abi.MOE_F16) == L.total


def test_timer_rejects_bad_capacity():
    h = ctypes.c_void_p()
    assert abi.lib().moe_timer_create(ctypes.byref(h), 0, 1) == 1
    assert abi.lib().moe_timer_create(ctypes.byref(h), 4, 0) == 1          # no stage selected
    assert abi.lib().moe_timer_create(ctypes.byref(h), 4, 1 << 8) == 1     # no such stage
    assert abi.lib().moe_timer_destroy(None) == 1


def _gpu_visible():
    import torch

    return torch.cuda.device_count() > 0


@pytest.mark.skipif(_gpu_visible(), reason="only meaningful on a machine without a GPU")
def test_no_device_gives_ehip_without_crash():
    # valid arguments, fake addresses, no GPU: the launch fails and the call reports it
    L = abi.lib()
    assert L.moe_combine(A, 64, A, 4, 2, 16, A, None) == 3


def test_route_rejects_bad_arguments():
    L = abi.lib()
    assert L.moe_route_topk(A, 4, 8, 9, A, A, None) == 1      # K > E
    assert L.moe_route_topk(A, 0, 8, 2, A, A, None) == 1      # T < 1
    assert L.moe_route_topk(A, 4, 2048, 8, A, A, None) == 2   # E too large
    assert L.moe_route_topk(A, 4, 512, 65, A, A, None) == 2   # K too large
    assert L.moe_route_topk(A + 2, 4, 8, 2, A, A, None) == 1  # misaligned


def test_noalloc_refuses_requests_beyond_its_buffer_before_any_hip_call():
    """the allocation-free forward has a fixed buffer of MOE_NOALLOC_WORKSPACE_BYTES:
    a larger request (the prefill shape needs ~454 MiB) is refused with
    MOE_ENOSPACE (4) on the host, like the other argument checks"""
    L = abi.lib()
    assert abi.NOALLOC_WORKSPACE_BYTES == 64 << 20
    assert "MOE_NOALLOC_WORKSPACE_BYTES (64u * 1024u * 1024u)" in open(HEADER).read()
    A = 1 << 20  # never dereferenced
    need = abi.moe_forward_workspace(2048, 10, 512, 2560, 768, 16, abi.MOE_F16)
    assert need > abi.NOALLOC_WORKSPACE_BYTES
    assert L.moe_forward_packed_noalloc(A, A, A, A, A, A, abi.MOE_F16, 2048, 10, 512, 2560, 768,
                                        16, A, None) == 4
    # bad sizes keep their own status
    assert L.moe_forward_packed_noalloc(A, A, A, A, A, A, abi.MOE_F16, 0, 10, 512, 2560, 768, 16,
                                        A, None) == 1
    assert L.moe_forward_packed_noalloc(A, A, A, A, A, A, abi.MOE_F16, 4, 8, 2000, 2816, 704, 16,
                                        A, None) == 2
    assert abi.moe_status_str(4).startswith("request larger than the fixed buffer")


def r256(v):
    return (v + 255) // 256 * 256


@pytest.mark.parametrize("T,K,E,d,f,dtype,packed,slots", [(4, 8, 128, 2816, 704, 2, 1, 0),
                                                          (4, 8, 128, 2816, 704, 2, 1, 64),
                                                          (64, 2, 8, 128, 256, 0, 0, 0),
                                                          (96, 2, 48, 328, 200, 1, 1, 48),
                                                          (3, 2, 1024, 64, 64, 0, 1, 0)])
def test_host_cache_bytes_closed_form(T, K, E, d, f, dtype, packed, slots):
    """the expert cache of moe_forward_host_weights: a 256-byte header, slot_of[E],
    exp_of[S], copy[S], then S slots of each matrix at the layout's per-expert size
    (S = slots, or min(E, T K) for 0), each region at a 256-byte boundary"""
    L = abi.lib()
    v = ctypes.c_size_t()
    es = 4 if dtype == 0 else 2
    if packed:
        assert L.moe_packed_weight_bytes(1, d, f, dtype, 0, ctypes.byref(v)) == 0
        bgu = v.value
        assert L.moe_packed_weight_bytes(1, d, f, dtype, 1, ctypes.byref(v)) == 0
        bdn = v.value
    else:
        bgu = bdn = d * f * es
    S = slots or min(E, T * K)
    off = r256(256 + E * 4)
    off = r256(off + S * 4)
    off = r256(off + S * 4)
    off = r256(off + S * bgu)
    off = r256(off + S * bgu)
    want = r256(off + S * bdn)
    assert L.moe_host_cache_bytes(T, K, E, d, f, dtype, packed, slots, ctypes.byref(v)) == 0
    assert v.value == want


def test_host_cache_calls_reject_bad_arguments():
    """sizes, slots and buffers are checked before any HIP call (the host
    pointers are only inspected once everything else is valid)"""
    L = abi.lib()
    v = ctypes.c_size_t()
    B = ctypes.byref(v)
    assert L.moe_host_cache_bytes(4, 8, 128, 2816, 704, 2, 2, 0, B) == 1     # packed = 2
    assert L.moe_host_cache_bytes(4, 9, 8, 64, 64, 1, 0, 0, B) == 1          # K > E
    assert L.moe_host_cache_bytes(4, 2, 8, 60, 64, 1, 0, 0, B) == 1          # d % 8
    assert L.moe_host_cache_bytes(4, 2, 2000, 64, 64, 1, 0, 0, B) == 2       # E too large
    assert L.moe_host_cache_bytes(4, 8, 128, 64, 64, 1, 0, 31, B) == 1       # slots < T K
    assert L.moe_host_cache_bytes(4, 8, 128, 64, 64, 1, 0, 129, B) == 1      # slots > E
    assert L.moe_host_cache_bytes(4, 8, 128, 64, 64, 1, 0, -1, B) == 1
    assert L.moe_host_cache_bytes(4, 2, 8, 64, 64, 1, 0, 0, None) == 1
    assert L.moe_host_cache_bytes(4, 2, 8, 64, 64, 1, 0, 8, B) == 0
    need = v.value
    A = 1 << 20  # made-up, never dereferenced addresses
    init = L.moe_host_cache_init
    assert init(A, need - 256, 8, 64, 64, 1, 0, 8, None) == 1                # small cache
    assert init(A + 16, need, 8, 64, 64, 1, 0, 8, None) == 1                 # misaligned
    assert init(None, need, 8, 64, 64, 1, 0, 8, None) == 1
    assert init(A, need, 8, 64, 64, 1, 0, 0, None) == 1                      # slots 0
    assert init(A, need, 8, 64, 64, 1, 0, 9, None) == 1                      # slots > E
    args = [A, A, A, A, A, A, 0, 1, 4, 2, 8, 64, 64, 16]
    fwd = L.moe_forward_host_weights
    assert fwd(*args, 8, A, need - 256, A, 1 << 30, A, None) == 1           # small cache
    assert fwd(*args, 8, A + 16, need, A, 1 << 30, A, None) == 1            # misaligned cache
    assert fwd(*args, 8, None, need, A, 1 << 30, A, None) == 1              # no cache
    assert fwd(*args, 7, A, need, A, 1 << 30, A, None) == 1                 # slots < min(E, TK)
    bad = list(args)
    bad[3] = None                                                           # no gate weights
    assert fwd(*bad, 8, A, need, A, 1 << 30, A, None) == 1
    bad = list(args)
    bad[6] = 3                                                              # packed = 3
    assert fwd(*bad, 8, A, need, A, 1 << 30, A, None) == 1
