"""The allocation-free entry point (ddh_exchange_staged_static) against the
entry point it stands in for (ddh_exchange_step with DDH_MODE_STAGED), bit
for bit, through the C ABI: two calls in a row on one process's static
staging buffer, the second on a smaller system; each pass alone; the size
limit; capture refusal; and no device memory taken by a warm call."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import domain_decomposition_halo_amd as ddh  # noqa: E402
import oracle  # noqa: E402
import workloads as W  # noqa: E402

pytestmark = pytest.mark.gpu


def bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def _system(k):
    w = W.WORKLOADS[k]
    x = W.positions(w)
    ref = oracle.OraclePlan(x, **w.params())
    plan = ddh.Plan(**w.params())
    xg = torch.from_numpy(x).cuda()
    lay = plan.build_maps(xg)
    return w, ref, plan, xg, lay


def _arrays(plan, xg, n_slots, f0):
    xl = torch.zeros((n_slots, 3), dtype=torch.float32, device="cuda")
    plan.gather_home(xg, xl)
    fl = torch.from_numpy(f0.copy()).cuda()
    return xl, fl


@pytest.mark.parametrize("first,second", [(2, 1), (4, 2)])
def test_static_staging_matches_the_staged_entry_point(first, second):
    for k in (first, second):
        w, ref, plan, xg, lay = _system(k)
        n = lay["n_slots"]
        f0 = W.forces(w, n)
        # the existing entry point: DDH_MODE_STAGED, staging allocated by the plan
        plan.set_mode(ddh.DDH_MODE_STAGED)
        xa, fa = _arrays(plan, xg, n, f0)
        plan.exchange_step(xa, fa)
        assert plan.check() == ddh.DDH_OK
        # the allocation-free one, with the plan left in its default mode
        plan.set_mode(ddh.DDH_MODE_AUTO)
        xb, fb = _arrays(plan, xg, n, f0)
        plan.exchange_staged_static(xb, fb)
        assert plan.check() == ddh.DDH_OK
        torch.cuda.synchronize()
        assert np.array_equal(bits(xb.cpu().numpy()), bits(xa.cpu().numpy())), k
        assert np.array_equal(bits(fb.cpu().numpy()), bits(fa.cpu().numpy())), k
        # and both are the oracle's
        fr = f0.copy()
        ref.exchange_forces(fr)
        assert np.array_equal(bits(xb.cpu().numpy()), bits(ref.x_local)), k
        assert np.array_equal(bits(fb.cpu().numpy()), bits(fr)), k
        # each pass alone, then a second step on the same buffers
        xc, fc = _arrays(plan, xg, n, f0)
        plan.exchange_staged_static(xc, None)
        plan.exchange_staged_static(None, fc)
        plan.exchange_staged_static(xc, fc)   # coordinates again (idempotent), forces twice
        fr2 = fr.copy()
        ref.exchange_forces(fr2)
        assert plan.check() == ddh.DDH_OK
        assert np.array_equal(bits(xc.cpu().numpy()), bits(ref.x_local)), k
        assert np.array_equal(bits(fc.cpu().numpy()), bits(fr2)), k
        plan.close()


def test_static_staging_allocates_nothing_when_warm():
    w, ref, plan, xg, lay = _system(3)
    n = lay["n_slots"]
    f0 = W.forces(w, n)
    xl, fl = _arrays(plan, xg, n, f0)
    plan.exchange_staged_static(xl, fl)   # warm: kernels loaded
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(3):
        plan.exchange_staged_static(xl, fl)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0
    assert plan.check() == ddh.DDH_OK
    plan.close()


def test_static_staging_limit_and_errors():
    # 12M atoms: 8.46M halo entries need 101 MB of staging, above the 64 MiB
    w, ref, plan, xg, lay = None, None, None, None, None
    w = W.WORKLOADS[5]
    plan = ddh.Plan(**w.params())
    xg = torch.from_numpy(W.positions(w)).cuda()
    lay = plan.build_maps(xg)
    assert 12 * lay["n_halo"] > ddh.DDH_STATIC_STAGE_BYTES
    xl = torch.zeros((lay["n_slots"], 3), dtype=torch.float32, device="cuda")
    with pytest.raises(ddh.DDHError) as e:
        plan.exchange_staged_static(xl, None)
    assert e.value.code == ddh.DDH_ECAPACITY
    assert "static" in ddh.last_error()
    with pytest.raises(ddh.DDHError) as e:
        plan.exchange_staged_static(None, None)
    assert e.value.code == ddh.DDH_EINVAL
    plan.close()
    # a small plan: buffers too small, overlapping arrays
    w2, ref2, p2, xg2, lay2 = _system(1)
    small = torch.zeros((lay2["n_slots"] - 1, 3), dtype=torch.float32, device="cuda")
    with pytest.raises(ddh.DDHError) as e:
        p2.exchange_staged_static(small, None)
    assert e.value.code == ddh.DDH_ECAPACITY
    big = torch.zeros((lay2["n_slots"], 3), dtype=torch.float32, device="cuda")
    with pytest.raises(ddh.DDHError) as e:
        p2.exchange_staged_static(big, big)
    assert e.value.code == ddh.DDH_EINVAL
    p2.close()


@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
def test_static_staging_refuses_capture():
    w, ref, plan, xg, lay = _system(1)
    n = lay["n_slots"]
    xl, fl = _arrays(plan, xg, n, W.forces(w, n))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with pytest.raises(ddh.DDHError) as e:
        with torch.cuda.graph(graph):
            plan.exchange_staged_static(xl, fl)
    assert e.value.code == ddh.DDH_EINVAL
    del graph
    torch.cuda.synchronize()
    plan.exchange_staged_static(xl, fl)
    assert plan.check() == ddh.DDH_OK
    assert np.array_equal(bits(xl.cpu().numpy()), bits(ref.x_local))
    plan.close()
