"""tq_decode_attention_noalloc against tq_decode_attention, through the C ABI.

The allocation-free entry point runs the same kernels with the workspace taken
from the library's fixed per-device scratch array, so its output must equal the
workspace entry point's bit for bit.  Two calls in a row, the second with a
smaller input (fewer sequences, shorter contexts), check that what the first
call left in the shared scratch does not leak into the second."""
import ctypes

import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _setup(wid, batch, T, hq=None):
    from kv_cache_online_amd.session import TQSession
    w0 = W.WORKLOADS[wid]
    w = W.small(w0, batch=batch, seq_len=T, **({"n_q_heads": hq} if hq else {}))
    rot, proj = W.rotation(w.d, w.wid), W.sketch(w.m, w.d, w.wid)
    s = TQSession(w.d, w.n_kv_heads, w.n_q_heads, rot, proj, k_bits=w.bits_mse, v_bits=w.bits_mse,
                  k_sketch=w.sketch, v_sketch=w.sketch)
    lens = np.full(batch, T, np.int64)
    starts = W.seq_starts(lens)
    kc, vc = s.new_caches(W.capacity(lens))
    dev = lambda a: (torch.from_numpy(np.ascontiguousarray(a)).cuda().view(torch.bfloat16)
                     if a.dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(a)).cuda())
    s.quantize(dev(W.kv_batch(w, 0)), dev(W.kv_batch(w, 1)), torch.from_numpy(starts).cuda(), kc, vc)
    q = dev(W.queries(w))
    return s, w, kc, vc, q, starts


def _both(s, w, kc, vc, q, starts, lens):
    from kv_cache_online_amd import binding as B
    st = torch.from_numpy(np.asarray(starts, np.int64)).cuda()
    ln = torch.from_numpy(np.asarray(lens, np.int32)).cuda()
    max_len = int(np.max(lens))
    ref = s.decode(q, st, ln, max_len, kc, vc)
    out = torch.full_like(ref, float("nan"))
    B.tq_decode_attention_noalloc(s.cfg, q, s.dtype_code(q), q.shape[0], st, ln, max_len, kc.desc, vc.desc,
                                  0.0, out, s.status)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), out.cpu().numpy()


@pytest.mark.parametrize("wid,hq", [(2, None), (3, None), (5, None), (2, 16)])
def test_noalloc_equals_workspace_decode_twice(wid, hq):
    """Matrix-core decode (workloads 2, 3, 5) and the reference kernels (16 query
    heads over 8 kv heads: G = 2)."""
    _need_gpu()
    s, w, kc, vc, q, starts = _setup(wid, 3, 2000, hq)
    ref, out = _both(s, w, kc, vc, q, starts, np.array([2000, 1500, 700]))
    assert np.isfinite(ref).all()
    np.testing.assert_array_equal(out, ref)
    # second call: fewer sequences, shorter contexts (the scratch holds the first call's data)
    ref2, out2 = _both(s, w, kc, vc, q[:2].contiguous(), starts[:2], np.array([300, 65]))
    np.testing.assert_array_equal(out2, ref2)
    assert int(s.status.item()) == 0


def test_noalloc_rejects_beyond_scratch():
    """A plan larger than the fixed scratch is refused before anything is enqueued."""
    _need_gpu()
    from kv_cache_online_amd import binding as B
    s, w, kc, vc, q, starts = _setup(2, 1, 64)
    big = 1 << 30
    need = B.tq_decode_workspace_bytes(s.cfg, 64, big)
    assert need > B.TQ_NOALLOC_SCRATCH_BYTES
    rc = B.LIB.tq_decode_attention_noalloc(ctypes.byref(s.cfg), q.data_ptr(), s.dtype_code(q), 64,
                                           q.data_ptr(), q.data_ptr(), big, ctypes.byref(kc.desc),
                                           ctypes.byref(vc.desc), 0.0, q.data_ptr(), None, None)
    assert rc == B.TQ_ERR_WORKSPACE
