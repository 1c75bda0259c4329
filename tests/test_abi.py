"""The C-ABI library loads, exports what include/verify_attn.h declares, and
rejects host-detectable errors with the documented codes (no GPU work)."""
import ctypes
import os
import re

import pytest

import mla_tree_verify_latent_amd as mtv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "verify_attn.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(verify_attn\w*)\s*\(", text)))


def header_enum(name):
    text = open(HEADER).read()
    m = re.search(rf"\b{name}\s*=\s*(-?\d+)", text)
    return int(m.group(1))


@pytest.fixture(scope="module")
def lib():
    return mtv.load_library()


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert set(names) == set(mtv.EXPORTS)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in the header but not exported"


def test_version(lib):
    assert mtv.verify_attn_version() == (1 << 16) | 6


def base_params(**kw):
    d = dict(num_seqs=1, num_heads=8, tree_size=64, max_seq_len=65600, total_kv=65600,
             pool_slots=131072, sm_scale=0.0721, nsplit=0)
    d.update(kw)
    return mtv.make_params(**d)


def test_workspace_and_plan():
    p = base_params()
    ws = mtv.verify_attn_workspace_size(p)
    plan = mtv.verify_attn_plan(p)
    M = 8 * 64
    assert plan["row_tiles"] == -(-M // plan["rows_per_tile"])
    assert plan["keys_per_split"] % 32 == 0
    assert plan["max_splits"] >= -(-65600 // plan["keys_per_split"])
    assert plan["partial_blocks"] % 8 == 0
    assert plan["partial_blocks"] >= plan["max_splits"] * plan["row_tiles"]
    assert ws == plan["max_splits"] * M * (512 * 2 + 2 * 4)  # bf16 V sums, fp32 (max, sum)
    # nsplit fixes the split length from max_seq_len
    p1 = base_params(nsplit=1)
    assert mtv.verify_attn_plan(p1)["keys_per_split"] >= 65600


@pytest.mark.parametrize("field,value,code", [
    ("num_seqs", 0, "VERIFY_ATTN_ERR_BAD_DIM"),
    ("num_heads", 0, "VERIFY_ATTN_ERR_BAD_DIM"),
    ("kv_dim", 512, "VERIFY_ATTN_ERR_BAD_DIM"),
    ("v_dim", 576, "VERIFY_ATTN_ERR_BAD_DIM"),
    ("tree_size", 0, "VERIFY_ATTN_ERR_TREE_TOO_LARGE"),
    ("tree_size", 65, "VERIFY_ATTN_ERR_TREE_TOO_LARGE"),
    ("max_seq_len", 63, "VERIFY_ATTN_ERR_BAD_SEQ"),
    ("total_kv", 63, "VERIFY_ATTN_ERR_BAD_SEQ"),
    ("total_kv", 65601, "VERIFY_ATTN_ERR_BAD_SEQ"),
    ("nsplit", -1, "VERIFY_ATTN_ERR_BAD_SPLIT"),
    ("pool_slots", 0, "VERIFY_ATTN_ERR_BAD_DIM"),
    ("page_size", 0, "VERIFY_ATTN_ERR_BAD_DIM"),
    ("reserved", 1, "VERIFY_ATTN_ERR_BAD_DIM"),
])
def test_param_errors(lib, field, value, code):
    p = base_params()
    setattr(p, field, value)
    assert mtv.verify_attn_workspace_size(p) == 0
    fake = 1 << 20
    rc = lib.verify_attn(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, 1 << 40, None)
    assert rc == header_enum(code)
    assert mtv.verify_attn_strerror(rc) not in ("ok", "unknown status")


def test_pointer_errors(lib):
    p = base_params()
    ws = mtv.verify_attn_workspace_size(p)
    a = 1 << 20
    args = [a, a, a, a, a, a, a]
    for i in range(7):
        bad = list(args)
        bad[i] = None
        rc = lib.verify_attn(ctypes.byref(p), *bad, ws, None)
        assert rc == header_enum("VERIFY_ATTN_ERR_NULL_PTR"), i
    for i in (0, 1, 5, 6):  # q, kv_pool, out, workspace must be 16-byte aligned
        bad = list(args)
        bad[i] = a + 8
        rc = lib.verify_attn(ctypes.byref(p), *bad, ws, None)
        assert rc == header_enum("VERIFY_ATTN_ERR_MISALIGNED"), i
    rc = lib.verify_attn(ctypes.byref(p), *args, ws - 1, None)
    assert rc == header_enum("VERIFY_ATTN_ERR_WORKSPACE_TOO_SMALL")
    rc = lib.verify_attn(None, *args, ws, None)
    assert rc == header_enum("VERIFY_ATTN_ERR_NULL_PTR")


def test_no_device_here(lib):
    """Valid arguments on a host without a gfx950 device: ERR_DEVICE, nothing launched."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a device is present; this checks the no-device path only")
    p = base_params()
    ws = mtv.verify_attn_workspace_size(p)
    a = 1 << 20
    rc = lib.verify_attn(ctypes.byref(p), a, a, a, a, a, a, a, ws, None)
    assert rc == header_enum("VERIFY_ATTN_ERR_DEVICE")


def test_strerror_total(lib):
    for code in range(-12, 2):
        assert isinstance(mtv.verify_attn_strerror(code), str)


def test_append_kv_errors(lib):
    """The draft-row append validates like the verify call and checks its own
    pointers before touching a device."""
    p = base_params()
    a = 1 << 20
    args = [a, a, a, a]  # kv_new, slot_idx, seq_lens, kv_pool
    for i in range(4):
        bad = list(args)
        bad[i] = None
        assert lib.verify_attn_append_kv(ctypes.byref(p), *bad, None) == header_enum("VERIFY_ATTN_ERR_NULL_PTR"), i
    for i in (0, 3):  # kv_new and kv_pool must be 16-byte aligned
        bad = list(args)
        bad[i] = a + 8
        assert lib.verify_attn_append_kv(ctypes.byref(p), *bad, None) == header_enum("VERIFY_ATTN_ERR_MISALIGNED"), i
    q = base_params(tree_size=0)
    assert lib.verify_attn_append_kv(ctypes.byref(q), *args, None) == header_enum("VERIFY_ATTN_ERR_TREE_TOO_LARGE")
    assert lib.verify_attn_append_kv(None, *args, None) == header_enum("VERIFY_ATTN_ERR_NULL_PTR")
    import torch
    if torch.cuda.device_count() == 0:
        assert lib.verify_attn_append_kv(ctypes.byref(p), *args, None) == header_enum("VERIFY_ATTN_ERR_DEVICE")


def test_compact_kv_errors(lib):
    """The KV compaction validates like the verify call and checks its own
    pointers before touching a device."""
    p = base_params()
    a = 1 << 20
    args = [a, a, a]  # kv_pool, slot_idx, kv_dst
    for i in range(3):
        bad = list(args)
        bad[i] = None
        assert lib.verify_attn_compact_kv(ctypes.byref(p), *bad, None) == header_enum("VERIFY_ATTN_ERR_NULL_PTR"), i
    for i in (0, 2):  # kv_pool and kv_dst must be 16-byte aligned
        bad = list(args)
        bad[i] = a + 8
        assert lib.verify_attn_compact_kv(ctypes.byref(p), *bad, None) == header_enum("VERIFY_ATTN_ERR_MISALIGNED"), i
    q = base_params(total_kv=0)
    assert lib.verify_attn_compact_kv(ctypes.byref(q), *args, None) != 0
    assert lib.verify_attn_compact_kv(None, *args, None) == header_enum("VERIFY_ATTN_ERR_NULL_PTR")
    import torch
    if torch.cuda.device_count() == 0:
        assert lib.verify_attn_compact_kv(ctypes.byref(p), *args, None) == header_enum("VERIFY_ATTN_ERR_DEVICE")


def test_f32_entry_errors(lib):
    """The fp32 entry point validates like the bf16 one and needs its own workspace size."""
    p = base_params()
    n32 = lib.verify_attn_f32_workspace_size(ctypes.byref(p))
    assert n32 > 0
    a = 1 << 20
    args = [a, a, a, a, a, a, a]  # q, kv, slot, lens, parent, out, ws
    for i in range(7):
        bad = list(args)
        bad[i] = None
        assert lib.verify_attn_f32(ctypes.byref(p), *bad, n32, None) == header_enum("VERIFY_ATTN_ERR_NULL_PTR"), i
    for i in (0, 1, 5, 6):
        bad = list(args)
        bad[i] = a + 8
        assert lib.verify_attn_f32(ctypes.byref(p), *bad, n32, None) == header_enum("VERIFY_ATTN_ERR_MISALIGNED"), i
    assert lib.verify_attn_f32(ctypes.byref(p), *args, n32 - 1, None) == header_enum(
        "VERIFY_ATTN_ERR_WORKSPACE_TOO_SMALL")
    import torch
    if torch.cuda.device_count() == 0:
        assert lib.verify_attn_f32(ctypes.byref(p), *args, n32, None) == header_enum("VERIFY_ATTN_ERR_DEVICE")


def test_noalloc_entry_errors(lib):
    """The allocation-free entry point validates like verify_attn, and refuses (before
    touching a device) a call whose partials exceed its scratch array."""
    p = base_params()
    a = 1 << 20
    args = [a, a, a, a, a, a]  # q, kv, slot, lens, parent, out
    for i in range(6):
        bad = list(args)
        bad[i] = None
        assert lib.verify_attn_noalloc(ctypes.byref(p), *bad, None) == header_enum("VERIFY_ATTN_ERR_NULL_PTR"), i
    for i in (0, 1, 5):
        bad = list(args)
        bad[i] = a + 8
        assert lib.verify_attn_noalloc(ctypes.byref(p), *bad, None) == header_enum("VERIFY_ATTN_ERR_MISALIGNED"), i
    scratch = int(re.search(r"VERIFY_ATTN_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)",
                            open(HEADER).read()).expand(r"\1 \2").split()[0]) << 20
    assert scratch == mtv.NOALLOC_SCRATCH_BYTES
    assert mtv.verify_attn_workspace_size(p) <= scratch  # the 64k-token H=8 shape fits
    big = mtv.make_params(num_seqs=4, num_heads=64, tree_size=64, max_seq_len=200768, total_kv=294400,
                          pool_slots=300000, sm_scale=0.07)
    assert mtv.verify_attn_workspace_size(big) > scratch
    assert lib.verify_attn_noalloc(ctypes.byref(big), *args, None) == header_enum("VERIFY_ATTN_ERR_SCRATCH_TOO_SMALL")
    import torch
    if torch.cuda.device_count() == 0:
        assert lib.verify_attn_noalloc(ctypes.byref(p), *args, None) == header_enum("VERIFY_ATTN_ERR_DEVICE")


def test_debug_validate_errors(lib):
    p = base_params()
    a = 1 << 20
    args = [a, a, a, a]  # slot_idx, seq_lens, tree_parent, flags
    for i in range(4):
        bad = list(args)
        bad[i] = None
        assert lib.verify_attn_debug_validate(ctypes.byref(p), *bad, None) == header_enum("VERIFY_ATTN_ERR_NULL_PTR"), i
    for i in range(4):
        bad = list(args)
        bad[i] = a + 2
        assert lib.verify_attn_debug_validate(ctypes.byref(p), *bad, None) == header_enum("VERIFY_ATTN_ERR_MISALIGNED"), i
    import torch
    if torch.cuda.device_count() == 0:
        assert lib.verify_attn_debug_validate(ctypes.byref(p), *args, None) == header_enum("VERIFY_ATTN_ERR_DEVICE")


def _check_plan_covers(plan, lens, H, T):
    c = plan["keys_per_split"]
    assert c % plan["keys_per_tile"] == 0 and c > 0
    splits = int(sum(-(-int(n) // c) for n in lens))
    assert splits <= plan["max_splits"], plan
    assert plan["partial_blocks"] >= plan["max_splits"] * plan["row_tiles"]
    assert plan["row_tiles"] * plan["rows_per_tile"] >= H * T


@pytest.mark.parametrize("cus,xcds", [(256, 8), (80, 2), (304, 8), (38, 1), (128, 4), (1, 1)])
def test_plan_under_other_device_shapes(cus, xcds):
    """The decomposition follows the device's compute units and XCDs: the grid is a
    multiple of the XCD count (workgroup ids are dealt to the XCDs round-robin), the
    automatic split length fills the given number of compute units, and every split
    is still covered, for both input types."""
    import numpy as np
    rng = np.random.default_rng(cus * 31 + xcds)
    for _ in range(60):
        B = int(rng.integers(1, 40))
        H = int(rng.choice([1, 8, 64]))
        T = int(rng.integers(1, 65))
        lens = rng.integers(T, T + int(rng.choice([1, 3000, 70000])), size=B)
        p = mtv.make_params(num_seqs=B, num_heads=H, tree_size=T, max_seq_len=int(lens.max()),
                            total_kv=int(lens.sum()), pool_slots=int(lens.sum()) + 1, sm_scale=0.07)
        for f32 in (False, True):
            plan = mtv.verify_attn_plan_for(p, f32, cus, xcds)
            assert plan["partial_blocks"] % xcds == 0
            _check_plan_covers(plan, lens, H, T)
    # one long sequence at H=8, T=64: the items fill the compute units in at most two rounds
    p = base_params()
    plan = mtv.verify_attn_plan_for(p, False, cus, xcds)
    items = -(-65600 // plan["keys_per_split"]) * plan["row_tiles"]
    assert items <= 2 * max(cus, plan["row_tiles"])
    assert items >= min(cus, 65600 // 256 * plan["row_tiles"]) * 0.75
    if cus == 256 and xcds == 8:
        assert plan == mtv.verify_attn_plan_for(p, False)  # no device here: a whole MI355X


def test_plan_rejects_bad_device_shape():
    p = base_params()
    for cus, xcds in [(8, 16), (-1, 1), (4, 0), (1 << 17, 8)]:
        with pytest.raises(mtv.VerifyAttnError):
            mtv.verify_attn_plan_for(p, False, cus, xcds)


def test_f32_plan_matches_its_workspace():
    p = base_params()
    plan = mtv.verify_attn_plan_for(p, True)
    assert plan["keys_per_tile"] == 16 and plan["rows_per_tile"] == 64
    # fp32 V sums and (max, sum) pairs
    assert mtv.verify_attn_f32_workspace_size(p) == plan["max_splits"] * 8 * 64 * (512 + 2) * 4


def test_plan_covers_every_split():
    """For random shapes and random valid sequence lengths (each in
    [tree_size, max_seq_len], summing to total_kv), the plan's max_splits and
    grid cover every (split, row tile) item the kernels derive on the device,
    and the combine's grid covers every output row."""
    import numpy as np
    rng = np.random.default_rng(7)
    for _ in range(400):
        B = int(rng.integers(1, 140))
        H = int(rng.choice([1, 2, 8, 16, 64]))
        T = int(rng.integers(1, 65))
        lens = rng.integers(T, T + int(rng.choice([1, 50, 3000, 70000])), size=B)
        max_len = int(lens.max()) + int(rng.choice([0, 0, 1, 999]))
        total = int(lens.sum())
        nsplit = int(rng.choice([0, 0, 0, 1, 3, 64]))
        p = mtv.make_params(num_seqs=B, num_heads=H, tree_size=T, max_seq_len=max_len, total_kv=total,
                            pool_slots=total + 5, sm_scale=0.07, nsplit=nsplit)
        plan = mtv.verify_attn_plan(p)
        c = plan["keys_per_split"]
        assert c % 32 == 0 and c > 0
        splits = int(sum(-(-int(n) // c) for n in lens))
        assert splits <= plan["max_splits"], (B, H, T, max_len, total, nsplit, plan)
        assert plan["partial_blocks"] >= plan["max_splits"] * plan["row_tiles"]
        assert plan["row_tiles"] * plan["rows_per_tile"] >= H * T
        # bf16 V sums [max_splits][H*T][512], then fp32 (max, sum) pairs
        assert mtv.verify_attn_workspace_size(p) == plan["max_splits"] * H * T * (512 * 2 + 2 * 4)
        assert mtv.verify_attn_f32_workspace_size(p) > 0


def test_split_length_overflow_rejected():
    """A split length that rounds past INT32_MAX (one split of a 2^31 - 1 token bound) is
    refused as invalid params instead of wrapping."""
    p = base_params(max_seq_len=2**31 - 1, total_kv=2**31 - 1, nsplit=1)
    assert mtv.verify_attn_workspace_size(p) == 0
    ok = base_params(max_seq_len=2**31 - 64, total_kv=2**31 - 64, nsplit=1)
    assert mtv.verify_attn_workspace_size(ok) > 0


def test_one_hip_runtime_whatever_the_import_order():
    """Loading the library before torch must not put a second HIP runtime in the
    process: torch's bundled runtime has the same soname as the system one, and the
    library has to bind to the copy that torch's tensors and streams belong to."""
    import subprocess
    import sys
    code = ("import mla_tree_verify_latent_amd as m; m.load_library(); import torch; "
            "paths = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}; "
            "print(len(paths))")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                         cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert out.returncode == 0, out.stderr[-2000:]
    assert out.stdout.strip().splitlines()[-1] == "1", out.stdout


def test_binding_refuses_tensors_on_another_device():
    """The binding's device check, as host logic (stand-in tensors and stream): tensors on
    two devices, or on a device other than the launch stream's, are refused before any
    pointer reaches the library."""
    import types
    import torch
    from mla_tree_verify_latent_amd import _check_device
    d0, d1 = torch.device("cuda", 0), torch.device("cuda", 1)
    def t(d):
        return types.SimpleNamespace(device=d)
    s0 = types.SimpleNamespace(device=d0)
    _check_device(s0, t(d0), t(d0), t(d0))
    with pytest.raises(ValueError, match="share one device"):
        _check_device(s0, t(d0), t(d1))
    with pytest.raises(ValueError, match="would run on"):
        _check_device(s0, t(d1), t(d1))


def test_plan_row_kernel_bands():
    """Rows per sequence pick the kernel: at most 32 the small-row kernel (64-key
    tiles, one row tile), more the 128-row kernel (32-key tiles). On a 256-CU
    device a call of at most 32 rows also takes the sliced combine (eight
    workgroups per row); more rows take at most two per row."""
    for H, T in [(1, 1), (8, 1), (8, 4), (4, 8), (16, 2), (3, 11), (8, 5), (8, 9), (16, 5), (8, 10),
                 (1, 64), (81, 1), (8, 11), (16, 8), (64, 64)]:
        M = H * T
        plan = mtv.verify_attn_plan(base_params(num_heads=H, tree_size=T))
        if M <= 32:
            assert plan["keys_per_tile"] == 64 and plan["row_tiles"] == 1 and plan["rows_per_tile"] == M, (H, T, plan)
            assert plan["combine_blocks"] == 8 * M, (H, T, plan)
        else:
            assert plan["keys_per_tile"] == 32 and plan["rows_per_tile"] == 128, (H, T, plan)
            assert plan["combine_blocks"] <= 2 * M, (H, T, plan)
