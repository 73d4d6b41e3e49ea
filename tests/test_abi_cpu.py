"""CPU: the C-ABI library loads, exports every declared symbol, computes the
same schedule as the independent re-derivation, and rejects bad arguments
before touching the GPU (no compute calls here)."""

import ctypes
import os
import re

import numpy as np
import pytest

import paged_kv_mla_amd as pk
from oracle.schedule_ref import (schedule_ref, flat_items, suffix_items, row_schedule_ref,
                                 kernel_config)
from mla_workloads import config_lens, CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    txt = open(os.path.join(ROOT, "include", "pkvmla.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(pkvmla_[a-z_0-9]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    syms = declared_symbols()
    assert len(syms) >= 10
    lib = ctypes.CDLL(pk.LIB_PATH)
    for s in syms:
        assert hasattr(lib, s), s
    assert sorted(pk.EXPORTED_SYMBOLS) == syms


@pytest.mark.parametrize("H", [16, 32, 64, 128])
def test_kernel_config_matches_table(H):
    lib = pk.kernel_config(H)
    ref = kernel_config(H)
    assert lib == {k: ref[k] for k in lib}


def test_kernel_config_rejects_other_head_counts():
    with pytest.raises(pk.PkvmlaError) as e:
        pk.kernel_config(48)
    assert e.value.code == pk.EUNSUPPORTED


def _compare(items, batch, num_wg, tile, fixed):
    w1, u1, m1 = pk.schedule_host(items, batch, num_wg, tile, fixed)
    w2, u2, m2 = schedule_ref(items, batch, num_wg, tile, fixed)
    np.testing.assert_array_equal(w1, w2)
    np.testing.assert_array_equal(u1, u2)
    np.testing.assert_array_equal(m1, m2)


@pytest.mark.parametrize("name", ["tiny", "deepseek", "long", "ragged"])
@pytest.mark.parametrize("num_cu", [256, 304, 80, 7, 1])
def test_schedule_host_matches_reference(name, num_cu):
    lens = config_lens(name)
    kc = kernel_config(CONFIGS[name]["num_heads"])
    _compare(flat_items(lens), len(lens), max(1, num_cu * kc["wg_per_cu"] // kc["head_groups"]),
             kc["tile"], kc["fixed_cost"])


def test_schedule_host_matches_reference_cascade():
    prefix, suffix = config_lens("cascade")
    B = len(suffix)
    _compare(suffix_items(1, suffix), B, 128, 32, 4)
    _compare(suffix_items(2, np.array([3, 0, 40, 0, 1])), 5, 512, 32, 1)


def _compare_rows(gi, pl, H, W):
    w1, u1, n1 = pk.schedule_rows_host(gi, pl, H, W)
    w2, u2, n2 = row_schedule_ref(gi, pl, H, W)
    np.testing.assert_array_equal(w1, w2)
    np.testing.assert_array_equal(u1, u2)
    assert n1 == n2


def test_row_schedule_host_matches_reference():
    prefix, suffix = config_lens("cascade")
    for H in (16, 32, 64, 128):
        for W in (256 // max(1, H // 64), 7, 1, 300):
            _compare_rows([0, len(suffix)], [prefix], H, W)
    _compare_rows([0, 2, 5], [64, 0], 16, 512)
    _compare_rows([0, 3], [100], 128, 2)
    rng = np.random.default_rng(11)
    for _ in range(150):
        G = int(rng.integers(1, 6))
        sizes = rng.integers(0, 9, size=G)
        gi = np.concatenate([[0], np.cumsum(sizes)])
        pl = rng.integers(0, 5000, size=G)
        _compare_rows(gi, pl, int(rng.choice([16, 32, 64, 128])), int(rng.integers(1, 400)))


def _compare_chain(gi, pl, kl, W):
    from oracle.schedule_ref import cascade_chain_ref
    w1, u1, m1, l1 = pk.schedule_chain_host(gi, pl, kl, W)
    r = cascade_chain_ref(gi, pl, kl, W)
    np.testing.assert_array_equal(w1, r["wg0"])
    np.testing.assert_array_equal(u1, r["units0"])
    np.testing.assert_array_equal(m1, r["merges"])
    np.testing.assert_array_equal(l1, r["slot_list"])


def test_chain_schedule_host_matches_reference():
    prefix, suffix = config_lens("cascade")
    for W in (128, 256, 64, 7, 1, 300):
        _compare_chain([0, len(suffix)], [prefix], suffix, W)
    rng = np.random.default_rng(12)
    for _ in range(150):
        G = int(rng.integers(1, 5))
        sizes = rng.integers(0, 7, size=G)
        sizes[0] = max(1, sizes[0])
        gi = np.concatenate([[0], np.cumsum(sizes)])
        pl = rng.integers(1, 3000, size=G)
        kl = rng.integers(0, 600, size=int(gi[-1]))
        _compare_chain(gi, pl, kl, int(rng.integers(1, 300)))


def test_row_schedule_host_rejects():
    with pytest.raises(pk.PkvmlaError):
        pk.schedule_rows_host([1, 2], [10], 16, 8)          # indptr[0] != 0
    with pytest.raises(pk.PkvmlaError):
        pk.schedule_rows_host([0, 2], [-1], 16, 8)          # negative prefix
    with pytest.raises(pk.PkvmlaError):
        pk.schedule_rows_host([0, 2], [10], 24, 8)          # heads not a multiple of 16


def test_schedule_host_random_cases():
    rng = np.random.default_rng(7)
    for _ in range(200):
        B = int(rng.integers(1, 40))
        lens = rng.integers(0, 3000, size=B)
        lens[rng.integers(0, B)] = max(1, lens.max())
        items = flat_items(lens)
        _compare(items, B, int(rng.integers(1, 600)), int(rng.choice([16, 32, 64])),
                 int(rng.integers(0, 4)))


# ---------------------------------------------------------------- validation
def _flat_args(**kw):
    a = dict(kv_indptr=[0, 2, 3], kv_indices=[0, 1, 2], kv_lens=[20, 5], num_heads=16,
             page_size=16, num_pages=4)
    a.update(kw)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(kv_indptr=[1, 2, 3]), pk.EINVAL),                 # indptr[0] != 0
    (dict(kv_indptr=[0, 3, 2]), pk.EINVAL),                 # non-monotone
    (dict(kv_lens=[0, 5]), pk.EINVAL),                      # empty request
    (dict(kv_indptr=[0], kv_indices=[], kv_lens=[]), pk.EINVAL),  # empty batch
    (dict(kv_lens=[33, 5]), pk.EINVAL),                     # more tokens than 2 pages hold
    (dict(kv_indices=[0, 9, 2]), pk.EINVAL),                # page id outside the pool
    (dict(kv_indices=[0, -1, 2]), pk.EINVAL),
    (dict(num_pages=0), pk.EINVAL),
    (dict(page_size=0), pk.EINVAL),
    (dict(page_size=24), pk.EUNSUPPORTED),                  # not a power of two
    (dict(page_size=512), pk.EUNSUPPORTED),
    (dict(num_heads=8), pk.EUNSUPPORTED),
    (dict(num_heads=1), pk.EUNSUPPORTED),
    (dict(ckv_dim=1), pk.EUNSUPPORTED),                     # head_dim_ckv = num_kv_heads mistake
    (dict(ckv_dim=256), pk.EUNSUPPORTED),
    (dict(kpe_dim=32), pk.EUNSUPPORTED),
    (dict(sm_scale=float("nan")), pk.EINVAL),
    (dict(sm_scale=float("inf")), pk.EINVAL),
    (dict(sm_scale=-0.5), pk.EINVAL),
    (dict(index_capacity=-1), pk.EINVAL),                   # negative page-id capacity
    (dict(index_capacity=2), pk.EINVAL),                    # below the table's 3 page ids
])
def test_plan_create_rejects(kw, code):
    with pytest.raises(pk.PkvmlaError) as e:
        pk.plan(**_flat_args(**kw))
    assert e.value.code == code
    assert pk.last_error()


def test_cascade_validation():
    base = dict(group_req_indptr=[0, 2], prefix_indptr=[0, 1], prefix_indices=[0],
                prefix_lens=[16], kv_indptr=[0, 1, 1], kv_indices=[1], kv_lens=[3, 0],
                num_heads=16, page_size=16, num_pages=4)
    for kw, code in [
        (dict(group_req_indptr=[0, 1]), pk.EINVAL),         # groups must cover the batch
        (dict(prefix_lens=[17]), pk.EINVAL),                # prefix longer than its page
        (dict(prefix_lens=[0]), pk.EINVAL),                 # request 1 would attend nothing
        (dict(kv_lens=[-1, 0]), pk.EINVAL),
        (dict(prefix_indices=[7]), pk.EINVAL),
    ]:
        a = dict(base)
        a.update(kw)
        with pytest.raises(pk.PkvmlaError) as e:
            pk.plan_cascade(**a)
        assert e.value.code == code, kw


def test_null_pointer_arguments_rejected():
    lib = ctypes.CDLL(pk.LIB_PATH)
    lib.pkvmla_run.argtypes = [ctypes.c_void_p] * 8
    assert lib.pkvmla_run(None, None, None, None, None, None, None, None) == pk.EINVAL
    lib.pkvmla_plan_destroy.argtypes = [ctypes.c_void_p]
    lib.pkvmla_plan_destroy(None)  # no-op
    lib.pkvmla_plan_create.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int32] * 6 + \
        [ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.pkvmla_plan_create(None, None, None, 1, 1, 16, 512, 64, 16, 0.0, None, None) == pk.EINVAL
    lib.pkvmla_plan_update.argtypes = [ctypes.c_void_p] * 5
    assert lib.pkvmla_plan_update(None, None, None, None, None) == pk.EINVAL


def test_package_without_library_fails_loudly(tmp_path):
    """No CPU or PyTorch fallback: the binding refuses to import without the
    built HIP library."""
    import shutil
    import subprocess
    import sys
    pkg = tmp_path / "paged_kv_mla_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "paged_kv_mla_amd", "__init__.py"), pkg / "__init__.py")
    code = ("import sys; sys.path.insert(0, %r)\n"
            "try:\n    import paged_kv_mla_amd\nexcept ImportError as e:\n"
            "    print('IMPORT_ERROR', e)\n") % str(tmp_path)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert "IMPORT_ERROR" in r.stdout and "no fallback" in r.stdout, r.stdout + r.stderr


def test_c_program_links_and_calls_host_entry_points(tmp_path):
    """The header is plain C99, and a C program links against the library and
    calls its host-only entry points (no GPU needed)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "abi.c"
    src.write_text(r'''
#include <stdio.h>
#include "pkvmla.h"
int main(void) {
  int32_t cfg[7];
  if (pkvmla_kernel_config(128, cfg) != PKVMLA_OK) return 1;
  if (pkvmla_kernel_config(8, cfg) != PKVMLA_EUNSUPPORTED) return 2;
  int32_t items[6] = {0, 0, 100, 1, 1, 40};
  int32_t wg[8], units[64], merges[16], counts[3];
  if (pkvmla_schedule_host(items, 2, 2, 4, 32, 1, wg, 8, units, 64, merges, 16, counts)) return 3;
  if (pkvmla_run(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL) != PKVMLA_EINVAL) return 4;
  printf("tile %d waves %d units %d %s\n", cfg[0], cfg[1], counts[1], pkvmla_last_error());
  return 0;
}
''')
    lib_dir = os.path.join(ROOT, "paged_kv_mla_amd")
    exe = tmp_path / "abi"
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                        f"-I{os.path.join(ROOT, 'include')}", str(src), "-o", str(exe),
                        f"-L{lib_dir}", "-lpkvmla", f"-Wl,-rpath,{lib_dir}"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert r.stdout.startswith("tile 32 waves 8 units")


# ------------------------------------------- binding-side argument checks
# The C layer sees raw pointers: sizes, devices and dtypes it cannot check are
# checked by the binding before any call (no GPU needed to see them refused).
@pytest.mark.parametrize("kw,msg", [
    (dict(kv_indptr=[0, 2]), "indptr needs 3"),             # one entry short
    (dict(kv_indptr=[0, 2, 3, 3]), "indptr needs 3"),       # one entry too many
    (dict(kv_indices=[0, 1]), "exceeds the 2 indices"),     # indptr[-1] = 3 > 2 ids
])
def test_plan_rejects_short_arrays(kw, msg):
    with pytest.raises(ValueError, match=msg):
        pk.plan(**_flat_args(**kw))


def test_plan_cascade_rejects_short_arrays():
    base = dict(group_req_indptr=[0, 2], prefix_indptr=[0, 1], prefix_indices=[0],
                prefix_lens=[16], kv_indptr=[0, 1, 1], kv_indices=[1], kv_lens=[3, 0],
                num_heads=16, page_size=16, num_pages=4)
    for kw, msg in [(dict(group_req_indptr=[0, 1, 2]), "num_groups"),
                    (dict(prefix_indptr=[0, 2]), "exceeds"),
                    (dict(kv_indptr=[0, 1]), "indptr needs"),
                    (dict(kv_indices=[]), "exceeds")]:
        a = dict(base)
        a.update(kw)
        with pytest.raises(ValueError, match=msg):
            pk.plan_cascade(**a)


def _fake_plan(B=2, H=16, ps=16, P=4):
    # handle 0: never passed to the library (every check below fails first)
    return pk.Plan(0, B, H, ps, P, 0)


def _tensors(B=2, H=16, ps=16, P=4, **over):
    import torch
    t = dict(q_nope=torch.zeros(B, H, 512, dtype=torch.bfloat16),
             q_pe=torch.zeros(B, H, 64, dtype=torch.bfloat16),
             ckv_cache=torch.zeros(P, ps, 512, dtype=torch.bfloat16),
             kpe_cache=torch.zeros(P, ps, 64, dtype=torch.bfloat16))
    t.update(over)
    return t


def test_run_rejects_bad_tensors_before_launch():
    import torch
    plan = _fake_plan()
    cases = [
        (dict(q_nope=torch.zeros(2, 16, 512, dtype=torch.float16)), "q_nope"),
        (dict(q_pe=torch.zeros(2, 8, 64, dtype=torch.bfloat16)), "q_pe"),
        (dict(ckv_cache=torch.zeros(3, 16, 512, dtype=torch.bfloat16)), "pages"),   # pool too small
        (dict(kpe_cache=torch.zeros(4, 8, 64, dtype=torch.bfloat16)), "pages"),     # page size
        (dict(out=torch.zeros(2, 16, 256, dtype=torch.bfloat16)), "out"),
        (dict(lse=torch.zeros(2, 16, dtype=torch.float16)), "lse"),
        (dict(), "cuda"),                                                          # CPU tensors
    ]
    for over, msg in cases:
        t = _tensors()
        out, lse = over.pop("out", None), over.pop("lse", None)
        t.update(over)
        if out is None:
            out = torch.zeros(2, 16, 512, dtype=torch.bfloat16)
        if lse is None:
            lse = torch.zeros(2, 16, dtype=torch.float32)
        with pytest.raises(ValueError, match=msg):
            plan.run(t["q_nope"], t["q_pe"], t["ckv_cache"], t["kpe_cache"], out=out, lse=lse)


@pytest.mark.parametrize("qo,code", [
    ([1, 2, 3], pk.EINVAL),            # qo_indptr[0] != 0
    ([0, 0, 1], pk.EINVAL),            # a request without query tokens
    ([0, 21, 22], pk.EINVAL),          # more query tokens than kv_len (20)
])
def test_plan_qo_rejects(qo, code):
    with pytest.raises(pk.PkvmlaError) as e:
        pk.plan_qo(qo, [0, 2, 3], [0, 1, 2], [20, 5], 16, 16, 4)
    assert e.value.code == code


def test_plan_qo_rejects_short_indptr():
    with pytest.raises(ValueError, match="qo_indptr"):
        pk.plan_qo([0, 1], [0, 2, 3], [0, 1, 2], [20, 5], 16, 16, 4)


def test_schedule_host_matches_reference_qo():
    from oracle.schedule_ref import qo_items
    qo = np.array([0, 2, 6, 7, 11])
    lens = np.array([40, 300, 1, 2000])
    _compare(qo_items(qo, lens), int(qo[-1]), 128, 32, 4)
    _compare(qo_items(qo, lens), int(qo[-1]), 7, 32, 2)


@pytest.mark.parametrize("seed", range(30))
def test_qo_row_schedule_host_matches_reference(seed):
    """The library's row-block schedule of several query tokens per request
    equals the independent re-derivation bit for bit (units, merges, slot
    list, slot count), and so does its layout rule."""
    from oracle.schedule_ref import qo_rows_ref, qo_uses_rows
    rng = np.random.default_rng(1000 + seed)
    H = int(rng.choice([16, 32]))
    B = int(rng.integers(1, 9))
    qo = rng.integers(1, 24 if seed % 3 else 3, size=B)
    kv = np.maximum(qo, rng.integers(1, 5000, size=B))
    qi = np.concatenate([[0], np.cumsum(qo)]).astype(np.int32)
    W = int(rng.choice([1, 3, 17, 64, 256]))
    fixed = int(rng.choice([1, 4]))
    got = pk.schedule_qo_rows_host(qi, kv, H, W, 32, fixed)
    ref = qo_rows_ref(qi, kv, H, W, 32, fixed)
    for g, r in zip(got[:4], ref[:4]):
        np.testing.assert_array_equal(g, r)
    assert got[4] == ref[4]
    assert got[5] == qo_uses_rows(qi, H)


@pytest.mark.parametrize("layout,H,code", [
    (7, 16, pk.EINVAL),                      # unknown layout
    (pk.QO_ROW_BLOCKS, 64, pk.EUNSUPPORTED),  # row blocks need 16 or 32 heads
    (pk.QO_ROW_BLOCKS, 128, pk.EUNSUPPORTED),
])
def test_plan_qo_layout_rejects(layout, H, code):
    with pytest.raises(pk.PkvmlaError) as e:
        pk.plan_qo([0, 2, 3], [0, 2, 3], [0, 1, 2], [20, 5], H, 16, 4, layout=layout)
    assert e.value.code == code


def test_qo_row_schedule_host_rejects():
    with pytest.raises(pk.PkvmlaError) as e:
        pk.schedule_qo_rows_host([0, 2], [10], 64, 8)
    assert e.value.code == pk.EUNSUPPORTED
    with pytest.raises(pk.PkvmlaError) as e:
        pk.schedule_qo_rows_host([0, 11], [10], 16, 8)      # more tokens than kv_len
    assert e.value.code == pk.EINVAL
