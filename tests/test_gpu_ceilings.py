"""GPU checks of the measurement helpers through the C ABI.

The random-row gather ceiling (dsa_ceiling_gather) leaves a checksum in its sink that depends
on exactly which bytes each thread moved, so both of its forms are checked bit for bit against
an emulation of its documented access pattern (index rows walked by workgroup, 32 listed rows
per chunk, piece p of a chunk moved by thread p % 512, out-of-range entries reading row 0).
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

NT, CH = 512, 32


def _dsa():
    import sparse_attention_long_gemm_amd as dsa
    dsa.load_library(build_if_missing=False)
    return dsa


def step(msg):
    print(f"\n[gpu step] {msg}", flush=True)


def _pieces(pool_i32, idx, qr, c, k, row16):
    """int32[NT, 4]: the 16-byte piece every thread moves as its k-th load of chunk c of index
    row qr."""
    n_rows = pool_i32.shape[0]
    pieces = row16 * CH
    p = np.arange(NT) + NT * k
    pp = np.where(p < pieces, p, 0)
    r, s = pp // row16, pp % row16
    rows = idx[qr, c + r].astype(np.int64)
    rows = np.where((rows >= 0) & (rows < n_rows), rows, 0)
    return pool_i32.reshape(n_rows, row16, 4)[rows, s]


def _expected(kind, pool_i32, idx, n_wg, row16):
    n_q, top_k = idx.shape
    per = (row16 * CH + NT - 1) // NT
    out = np.zeros((n_wg, NT), dtype=np.float32)
    for b in range(n_wg):
        acc = np.zeros((NT, 4), dtype=np.int32)
        last_even = None   # kind 0: buffer 0 of each wave holds its last even-numbered wave-load
        n = 0
        for qr in range(b, n_q, n_wg):
            for c in range(0, top_k - CH + 1, CH):
                for k in range(per):
                    x = _pieces(pool_i32, idx, qr, c, k, row16)
                    if kind == 1:
                        acc ^= x
                    elif n % 2 == 0:
                        last_even = x
                    n += 1
        if kind == 1:
            v = acc[:, 0] ^ acc[:, 1] ^ acc[:, 2] ^ acc[:, 3]
        else:
            # thread (wave, lane) reads int `lane` of its wave's buffer 0, which lane l of the
            # wave's last even wave-load filled with 16 bytes at offset 16 l
            v = np.empty(NT, dtype=np.int32)
            for t in range(NT):
                w, lane = t // 64, t % 64
                v[t] = last_even[64 * w + lane // 4, lane % 4]
        out[b] = v.astype(np.float32)
    return out.reshape(-1)


@pytest.mark.parametrize("kind", [0, 1])
def test_ceiling_gather_moves_the_listed_rows(kind):
    dsa = _dsa()
    step(f"dsa_ceiling_gather kind {kind}: 50 rows of 1152 bytes, 5 index rows of 64, 2 workgroups")
    rng = np.random.default_rng(7)
    n_rows, row_bytes, n_q, top_k, n_wg = 50, 1152, 5, 64, 2
    pool = rng.integers(-2**31, 2**31 - 1, size=(n_rows, row_bytes // 4), dtype=np.int64).astype(np.int32)
    idx = rng.integers(-3, n_rows + 5, size=(n_q, top_k)).astype(np.int32)   # some out of range
    dev = torch.device("cuda:0")
    pool_t = torch.from_numpy(pool).to(dev)
    idx_t = torch.from_numpy(idx).to(dev)
    sink = torch.full((n_wg * NT,), -1.0, dtype=torch.float32, device=dev)
    nb = dsa.ceiling_gather(kind, pool_t, idx_t, n_wg, sink)
    torch.cuda.synchronize()
    assert nb == n_q * top_k * row_bytes
    want = _expected(kind, pool, idx, n_wg, row_bytes // 16)
    got = sink.cpu().numpy()
    assert np.array_equal(got, want), f"{int((got != want).sum())} of {got.size} sink values differ"
