"""hga_decode_step_noalloc (scratch in the library's fixed per-device array,
nothing allocated) against hga_decode_step_ex (caller workspace), called
through the C ABI: two calls in a row on one device, the second with a
smaller input (three calls, each smaller than the one before), each with
outputs the caller allocated beforehand."""
import ctypes

import pytest
import torch

import hierarchical_sparse_attention_summaries_amd as hga
from synth import DECODE_64K, generate
from tests.gpu_runner import log, to_dev

pytestmark = pytest.mark.gpu

# batch 16 runs as two launches (refreshing route, then attention), the others
# as one
B16 = DECODE_64K.with_(name="noalloc-b16-t4096", B=16, T=4096, k_chunk=2, k_group=4, plants=1)
BIG = DECODE_64K.with_(name="noalloc-b2-t16384", B=2, T=16384, k_chunk=8, k_group=16, plants=2)
SMALL = DECODE_64K.with_(name="noalloc-b1-t4096", B=1, Hq=8, Hkv=2, T=4096, k_chunk=2,
                         k_group=4, plants=1)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _prepare(w):
    inp = generate(w)
    Q, K, V = (to_dev(x, w.dtype) for x in (inp.Q, inp.K, inp.V))
    cm, gm = hga.build_summaries(K, w.chunk, w.group)
    K[:, :, -1] += 0.75            # the newest key changed after the summaries were built
    return Q, K, V, cm, gm


def _outputs(w, Q):
    dev = Q.device
    return (torch.empty_like(Q), torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=dev),
            torch.empty((w.B, w.Hq, w.Nq, w.k_chunk + 2), dtype=torch.int32, device=dev),
            torch.empty((w.B, w.Hq, w.Nq, w.k_group), dtype=torch.int32, device=dev))


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def test_noalloc_matches_decode_step_ex_twice_smaller_second():
    L = hga.lib()
    for w in (B16, BIG, SMALL):
        log(f"case {w.name}")
        Q, K, V, cm, gm = _prepare(w)
        shape = hga.Shape(w.B, w.Hq, w.Hkv, w.Nq, w.T, w.D)
        # reference: the workspace form
        cm_r, gm_r = cm.clone(), gm.clone()
        O_r, lse_r, c_r, g_r = hga.decode_step_ex(Q, K, V, cm_r, gm_r, w.T, w.chunk, w.group,
                                                  w.k_chunk, w.k_group)
        # the allocation-free form, through the raw C ABI, on buffers made beforehand
        O, lse, c, g = _outputs(w, Q)
        cm_n, gm_n = cm.clone(), gm.clone()
        torch.cuda.synchronize()
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        st = L.hga_decode_step_noalloc(ctypes.byref(shape), None, _p(Q), _p(K), _p(V), 1,
                                       _p(cm_n), _p(gm_n), w.chunk, w.group, w.k_chunk,
                                       w.k_group, ctypes.c_float(0.0), _p(c), _p(g), _p(O),
                                       _p(lse), 0, stream)
        assert st == 0, hga.HGAError(st, "hga_decode_step_noalloc")
        torch.cuda.synchronize()
        # same kernels and plans on the same inputs: the same bits
        assert torch.equal(c, c_r) and torch.equal(g, g_r)
        assert torch.equal(cm_n, cm_r) and torch.equal(gm_n, gm_r)
        assert torch.equal(O, O_r) and torch.equal(lse, lse_r)
        assert bool(torch.isfinite(lse).all())
