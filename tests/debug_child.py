"""Child process of test_gpu_debug.py: runs on the library KV4_LIBRARY names
(the -DKV4_DEBUG build) and prints one JSON line per case with the
kv4_debug_flags bits the case raised and whether its outputs are finite.
Every bad input here is one the kernels' own bounds checks absorb (clamped or
skipped): none reaches memory outside the buffers."""
import json
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import paged_decode_attention_reshape_amd as kv4  # noqa: E402
import workloads as W  # noqa: E402

DEV = torch.device("cuda:0")


def setup(name, nq, nkv, hs, ql, sl):
    w = W.custom(name, nq, nkv, hs, ql, sl, block_size=16)
    lay = W.make_layout(w)
    t = W.make_tensors(w, lay)
    slots = torch.from_numpy(W.all_slots(lay, w)).to(DEV)
    nb = lay.num_blocks
    kc = torch.zeros((nb, 16, nkv, hs // 2), dtype=torch.uint8, device=DEV)
    vc = torch.zeros_like(kc)
    ks = torch.zeros((nb, 16, nkv), dtype=torch.float32, device=DEV)
    vs = torch.zeros_like(ks)
    return w, lay, t, slots, (kc, vc, ks, vs)


def attend(w, lay, t, caches, bt=None, sl=None, qsl=None):
    kc, vc, ks, vs = caches
    bt = torch.from_numpy(lay.block_table if bt is None else bt).to(DEV)
    sl = torch.from_numpy(lay.seq_lens if sl is None else sl).to(DEV)
    qsl = torch.from_numpy(lay.query_start_loc if qsl is None else qsl).to(DEV)
    return kv4.kv4_paged_attention(t.query.to(DEV), kc, vc, ks, vs, bt, sl, qsl, max_query_len=w.max_query_len,
                                   max_seq_len=w.max_seq_len, sign_seed=w.sign_seed)


def debug_flags(clear):
    # -1 on a release library (kv4_debug_flags: KV4_EUNSUPPORTED)
    try:
        return kv4.kv4_debug_flags(clear=clear)
    except kv4.Kv4Error as e:
        if e.code != kv4.KV4_EUNSUPPORTED:
            raise
        return -1


def case(name, fn):
    debug_flags(True)
    finite, extra = fn()
    flags = debug_flags(True)
    print(json.dumps({"case": name, "flags": flags, "finite": bool(finite), **extra}), flush=True)


def main():
    mode = sys.argv[1]
    cases = [("valid_decode", 32, 8, 128, [1] * 4, [1000, 17, 300, 2049]),
             ("valid_prefill", 12, 2, 128, [40, 1, 300], [100, 64, 900]),
             ("valid_hs96", 8, 8, 96, [1, 3], [400, 33])]
    outs = {}
    for name, nq, nkv, hs, ql, sl in cases:
        w, lay, t, slots, caches = setup(name, nq, nkv, hs, ql, sl)

        def run():
            kv4.kv4_rht_write(t.key.to(DEV), t.value.to(DEV), *caches, slots, sign_seed=w.sign_seed)
            o = attend(w, lay, t, caches)
            torch.cuda.synchronize()
            outs[name] = o.float().cpu().numpy()
            return torch.isfinite(o).all().item(), {}
        case(name, run)
    if mode == "valid":
        np.savez(sys.argv[2], **outs)
        return
    # bad inputs, one kind per case
    w, lay, t, slots, caches = setup("bad", 16, 4, 128, [1, 1, 1], [500, 300, 40])

    def bad_slot():
        s = slots.clone()
        s[3] = lay.num_blocks * 16 + 5        # past the cache: skipped
        kv4.kv4_rht_write(t.key.to(DEV), t.value.to(DEV), *caches, s, sign_seed=w.sign_seed)
        return True, {}
    case("bad_slot", bad_slot)
    kv4.kv4_rht_write(t.key.to(DEV), t.value.to(DEV), *caches, slots, sign_seed=w.sign_seed)
    debug_flags(True)

    def bad_page():
        bt = lay.block_table.copy()
        bt[0, 2] = lay.num_blocks + 3         # masked as no data
        o = attend(w, lay, t, caches, bt=bt)
        torch.cuda.synchronize()
        return torch.isfinite(o).all().item(), {}
    case("bad_page", bad_page)

    def bad_seqlen():
        sl = lay.seq_lens.copy()
        sl[1] = lay.block_table.shape[1] * 16 + 100   # beyond the page table: clamped
        o = attend(w, lay, t, caches, sl=sl)
        torch.cuda.synchronize()
        return torch.isfinite(o).all().item(), {}
    case("bad_seqlen", bad_seqlen)

    def bad_qsl():
        q = lay.query_start_loc.copy()
        q[2] = q[3] + 1                        # decreasing after it: clamped
        o = attend(w, lay, t, caches, qsl=q)
        torch.cuda.synchronize()
        return torch.isfinite(o).all().item(), {}
    case("bad_qsl", bad_qsl)


if __name__ == "__main__":
    main()
