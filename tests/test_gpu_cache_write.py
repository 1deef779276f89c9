"""GPU parity of the cache write (dsa_cache_append) through the C ABI, against the oracle.

* the FP8 quantisation of every bf16 bit pattern, byte for byte;
* whole caches after appends (one token per sequence, and a chunk of tokens with a sequence
  map, including rows with invalid slots), byte for byte;
* the decode step then runs on the written caches and matches the oracle's decode on the
  oracle-written caches.
"""
import numpy as np
import pytest
import torch

from gen import inputs as gi
from oracle import dsa_oracle as orc

from gates import check_attn, check_idx

pytestmark = pytest.mark.gpu


def _dsa():
    import sparse_attention_long_gemm_amd as dsa
    dsa.load_library(build_if_missing=False)
    return dsa


def step(msg):
    print(f"\n[gpu step] {msg}", flush=True)


def test_cache_append_quantises_every_bf16_value():
    """512 rows of 128 keys hold all 65536 bf16 patterns (NaNs, infinities, subnormals, ties)."""
    dsa = _dsa()
    T, d_I, P = 512, 128, 64
    k_new = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    k_new = k_new.reshape(T, d_I).contiguous()
    n_pages = T // P
    pt = torch.arange(n_pages, dtype=torch.int32)[None, :]
    seq = torch.zeros(T, dtype=torch.int32)
    pos = torch.arange(T, dtype=torch.int32)
    kc = torch.zeros((n_pages, P, d_I), dtype=torch.uint8, device="cuda")
    step("cache append: quantise all 65536 bf16 patterns")
    dsa.cache_append(pt.cuda(), pos.cuda(), k_cache=kc, k_new=k_new.cuda(), seq=seq.cuda())
    torch.cuda.synchronize()
    want = orc.quantize_e4m3fn(k_new.double().numpy()).reshape(n_pages, P, d_I)
    got = kc.cpu().numpy()
    bad = np.flatnonzero(got.reshape(-1) != want.reshape(-1))
    assert bad.size == 0, (f"{bad.size} codes differ, first bf16 patterns "
                           f"{[hex(int(x)) for x in bad[:6]]}")


def test_cache_append_rows_and_chunks_byte_exact():
    dsa = _dsa()
    g = torch.Generator().manual_seed(71)
    P, n_pages, d_I, D_k, B, max_pages = 64, 50, 128, 576, 5, 9
    perm = torch.randperm(n_pages, generator=g).to(torch.int32)
    pt = perm[: B * max_pages].reshape(B, max_pages).clone()
    pt[4, 6:] = -1
    kc = torch.randint(0, 256, (n_pages, P, d_I), generator=g, dtype=torch.int32).to(torch.uint8)
    kvc = torch.randn((n_pages, P, D_k), generator=g).to(torch.bfloat16)
    # a decode-style append (row r -> sequence r) then a chunk of 300 tokens of sequence 2 plus
    # rows with invalid slots (position past the table, negative, on a -1 page)
    pos1 = torch.tensor([0, 63, 64, 575, 383], dtype=torch.int32)
    seq2 = torch.tensor([2] * 300 + [1, 3, 4], dtype=torch.int32)
    pos2 = torch.tensor(list(range(100, 400)) + [576, -1, 400], dtype=torch.int32)
    kc_g, kvc_g = kc.cuda(), kvc.cuda()
    ref_k, ref_kv = kc.numpy(), kvc.view(torch.int16).numpy()
    for seq, pos in ((None, pos1), (seq2, pos2)):
        T = pos.shape[0]
        k_new = (torch.randn((T, d_I), generator=g) * 4).to(torch.bfloat16)
        kv_new = torch.randn((T, D_k), generator=g).to(torch.bfloat16)
        step(f"cache append: {T} rows, seq map {'yes' if seq is not None else 'no'}")
        dsa.cache_append(pt.cuda(), pos.cuda(), k_cache=kc_g, kv_cache=kvc_g,
                         k_new=k_new.cuda(), kv_new=kv_new.cuda(),
                         seq=None if seq is None else seq.cuda())
        torch.cuda.synchronize()
        ref_k, ref_kv = orc.cache_append(ref_k, ref_kv, pt, seq, pos, k_new, kv_new)
        assert np.array_equal(kc_g.cpu().numpy(), ref_k)
        assert np.array_equal(kvc_g.view(torch.int16).cpu().numpy(), ref_kv)


def test_decode_step_on_appended_caches():
    """The new token of each sequence (position ctx-1) is written by the append kernel into
    caches whose slot held other values; the decode step then reads it from there."""
    dsa = _dsa()
    sp = gi.DecodeSpec(B=6, idx=gi.IndexerSpec(top_k=512), mqa=gi.MqaSpec(sigma=1.0),
                       spare_pages=3, seed=73)
    d = gi.decode_inputs(sp, ctx_lens=(3000, 700, 2049, 513, 64, 1))
    B = 6
    g = torch.Generator().manual_seed(74)
    # new keys on the dyadic grid (exact scores), new KV rows N(0, 1)
    k_new = (torch.randint(-2, 3, (B, 128), generator=g).float() / 8).to(torch.bfloat16)
    kv_new = torch.randn((B, 576), generator=g).to(torch.bfloat16)
    pos = (d["ctx"] - 1).to(torch.int32)
    gd = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in d.items()}
    step("decode on appended caches: append")
    dsa.cache_append(gd["page_table"], pos.cuda(), k_cache=gd["k_cache"],
                     kv_cache=gd["kv_cache"], k_new=k_new.cuda(), kv_new=kv_new.cuda())
    step("decode on appended caches: indexer + MQA")
    idx = dsa.indexer_topk_paged(gd["q_idx"], gd["w"], gd["k_cache"], gd["page_table"],
                                 gd["ctx"], d["top_k"])
    o, lse = dsa.sparse_mqa_decode(gd["q"], gd["kv_cache"], gd["page_table"], gd["ctx"], idx,
                                   d["D_v"], d["scale"])
    torch.cuda.synchronize()
    kc, kvc = orc.cache_append(d["k_cache"], d["kv_cache"], d["page_table"], None, pos, k_new,
                               kv_new)
    d_ref = dict(d, k_cache=kc, kv_cache=kvc)
    i_ref, o_ref, l_ref = orc.decode(d_ref)
    check_idx(idx, i_ref, "decode idx on appended caches")
    check_attn(o, lse, o_ref, l_ref, "decode attn on appended caches")
    assert (i_ref == (pos.numpy()[:, None])).any(axis=1).sum() >= 1   # a new token was picked
