"""The allocation-free attention entry point (static device scratch) against
the one that takes a caller workspace: identical output bits on two calls in
a row, the second smaller, through the C ABI; and its size limit."""

import sys

import numpy as np
import pytest

from oracle import attention as oattn, codec
import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
ecco = pytest.importorskip("entropy_coded_group_amd")


def say(msg):
    print("[gpu-noalloc] " + msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    name = torch.cuda.get_device_properties(0).gcnArchName
    if not name.startswith("gfx950"):
        pytest.skip("not gfx950: %s" % name)
    ecco.lib()
    return torch.device("cuda:0")


def _tables(kind):
    blob = ecco.ecco_train_patterns(W.kv_sample(kind), threads=8)
    c, l = ecco.ecco_tables_get(blob)
    t = ecco.ecco_tensor_scale_from_amax(float(np.max(np.abs(W.kv_sample(kind).numpy().astype(np.float32)))))
    return codec.Tables(c, l), ecco.tables_to_device(blob), np.float32(t)


def _case(B, H, G, S, stride, seed, tk, tv):
    (tbk, tdk, sk), (tbv, tdv, sv) = tk, tv
    k = W.kv_tensor("k", shape=(B, H, stride, 128), seed=seed).numpy()
    v = W.kv_tensor("v", shape=(B, H, stride, 128), seed=seed + 1).numpy()
    kb = codec.encode_groups(k.reshape(-1, 128), tbk, sk).reshape(B, H, stride, 64)
    vb = codec.encode_groups(v.reshape(-1, 128), tbv, sv).reshape(B, H, stride, 64)
    q = W.c5_x(B * H * G, 128, seed=seed + 2).numpy().reshape(B, H * G, 128)
    return dict(B=B, H=H, G=G, S=S, stride=stride, kb=kb, vb=vb, q=q, kd=torch.from_numpy(kb).cuda(),
                vd=torch.from_numpy(vb).cuda(), qd=torch.from_numpy(q).cuda(), tdk=tdk, tdv=tdv, sk=sk, sv=sv,
                tbk=tbk, tbv=tbv)


def test_noalloc_attention_matches_workspace_attention_twice(dev):
    tk, tv = _tables("k"), _tables("v")
    cases = [_case(2, 4, 4, 1000, 1024, 31, tk, tv), _case(1, 2, 2, 77, 80, 41, tk, tv)]
    for n, c in enumerate(cases):
        B, H, G, S, st = c["B"], c["H"], c["G"], c["S"], c["stride"]
        scale = 1.0 / np.sqrt(128.0)
        ws = torch.empty(ecco.ecco_attention_workspace_size(B, H, G, S), dtype=torch.uint8, device="cuda")
        ref = torch.full((B, H * G, 128), float("nan"), dtype=torch.float32, device="cuda")
        got = torch.full((B, H * G, 128), float("nan"), dtype=torch.float32, device="cuda")
        say("call %d: B=%d H=%d G=%d S=%d" % (n, B, H, G, S))
        ecco.ecco_attention_decode(c["kd"], c["tdk"], c["sk"], c["vd"], c["tdv"], c["sv"], c["qd"], B, H, G, S, st,
                                   scale, ws, ref)
        ecco.ecco_attention_decode_noalloc(c["kd"], c["tdk"], c["sk"], c["vd"], c["tdv"], c["sv"], c["qd"], B, H, G,
                                           S, st, scale, got)
        torch.cuda.synchronize()
        r, g = ref.cpu().numpy(), got.cpu().numpy()
        assert not np.any(np.isnan(g))
        assert np.array_equal(r.view(np.uint32), g.view(np.uint32)), "call %d differs" % n
        # and within the oracle's tolerance on one (sequence, kv head) pair
        kd = codec.decode_blocks(c["kb"][0, 0, :S].reshape(-1, 64), c["tbk"], c["sk"]).reshape(1, 1, S, 128)
        vd = codec.decode_blocks(c["vb"][0, 0, :S].reshape(-1, 64), c["tbv"], c["sv"]).reshape(1, 1, S, 128)
        want, mag = oattn.attention_ref(kd, vd, c["q"][0:1, :G], scale)
        ok, worst = oattn.attention_tolerance_ok(g[0:1, :G], want, mag)
        assert ok, "call %d: worst error / bound %g" % (n, worst)
