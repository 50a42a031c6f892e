"""Helpers for the GPU parity tests: host arrays <-> device tensors, pool setup."""
import numpy as np

from cross_model_shared_amd import binding
from cross_model_shared_amd import workload as wlmod

POISON_BIG = 0x4480   # bf16 1024.0: a wrongly read slot dominates any score/value
POISON_NAN = 0x7FC0   # bf16 quiet NaN: a wrongly read slot poisons the output


def dev_bf16(bits: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).cuda().view(
        torch.bfloat16)


def dev_i32(x):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def host_bits(t) -> np.ndarray:
    import torch

    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f64(t) -> np.ndarray:
    import torch

    return t.detach().float().cpu().numpy().astype(np.float64)


def pool_bits(pool: binding.Pool) -> np.ndarray:
    return pool.data.cpu().numpy().view(np.uint16)


def status_tensor():
    import torch

    return torch.zeros(1, dtype=torch.int32, device="cuda")


def sync():
    import torch

    torch.cuda.synchronize()


def nan_workspace(nbytes):
    """A decode workspace whose every byte past the arrival counters is 0xFF (NaN as
    floats): the library must not read a byte of it that the same call has not
    written.  The counters are zeroed by shared_kv_decode_workspace_init, as the
    header asks before a workspace's first call."""
    import torch

    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    binding.decode_workspace_init(ws)
    return ws


def make_decode_case(lens, N, Hkv, G, D, seed, std=1.0, layers=1, layer=0, poison=POISON_BIG,
                     spare_frac=0.05):
    """Pool (GPU, via kv_pool_append) holding each session's logical K/V, plus queries.

    Returns a dict with host arrays (bits) for the oracle and device tensors.
    """
    rng = np.random.default_rng(seed)
    bt, num_pages = wlmod.build_block_table(lens, seed, spare_frac=spare_frac)
    K = [wlmod.draw_bf16(rng, (L, Hkv, D), std) for L in lens]
    V = [wlmod.draw_bf16(rng, (L, Hkv, D), std) for L in lens]
    q = wlmod.draw_bf16(rng, (len(lens), N, Hkv * G, D), std)
    kk, cu = wlmod.concat_rows(K)
    vv, _ = wlmod.concat_rows(V)
    pool = binding.Pool(layers, num_pages, Hkv, D, fill=np.int16(np.uint16(poison).view(np.int16)))
    st = status_tensor()
    max_len = max(max(lens), 1)
    if kk.shape[0]:
        binding.append(pool, layer, dev_bf16(kk), dev_bf16(vv), dev_i32(cu), dev_i32(bt),
                       dev_i32(np.zeros(len(lens))), max_new=max_len, max_seq_len=max_len, dev_status=st)
    return dict(lens=list(lens), N=N, Hkv=Hkv, G=G, D=D, bt=bt, num_pages=num_pages, K=K, V=V, q=q,
                kk=kk, vv=vv, cu=cu, pool=pool, status=st, layers=layers, layer=layer, poison=poison)


def run_decode(case, q_bits=None, lens=None, bt=None, max_seq_len=None, scale=None):
    import torch

    q_bits = case["q"] if q_bits is None else q_bits
    lens = case["lens"] if lens is None else lens
    bt = case["bt"] if bt is None else bt
    B, N, Hq, D = q_bits.shape
    msl = max(max(lens), 1) if max_seq_len is None else max_seq_len
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    ws = nan_workspace(binding.decode_workspace_bytes(B, N, Hq, case["Hkv"], D, msl))
    out = torch.empty((B, N, Hq, D), dtype=torch.bfloat16, device="cuda")
    binding.decode(case["pool"], case["layer"], dev_bf16(q_bits), out, dev_i32(bt), dev_i32(lens), msl,
                   scale, ws, dev_status=case["status"])
    sync()
    return out


def make_private_case(lens, priv, N, Hkv, G, D, seed, poison=POISON_NAN, std=1.0):
    """Pool (GPU) with B shared prefixes and B*N private suffixes, appended with
    kv_pool_append through the two block tables; logical K/V kept for the oracle."""
    rng = np.random.default_rng(seed)
    bt, pbt, num_pages = wlmod.build_private_tables(lens, priv, seed, spare_frac=0.05)
    K = [wlmod.draw_bf16(rng, (L, Hkv, D), std) for L in lens]
    V = [wlmod.draw_bf16(rng, (L, Hkv, D), std) for L in lens]
    Kp = [wlmod.draw_bf16(rng, (U, Hkv, D), std) for U in priv]
    Vp = [wlmod.draw_bf16(rng, (U, Hkv, D), std) for U in priv]
    q = wlmod.draw_bf16(rng, (len(lens), N, Hkv * G, D), std)
    pool = binding.Pool(1, num_pages, Hkv, D, fill=np.int16(np.uint16(poison).view(np.int16)))
    st = status_tensor()
    for table, ks, vs, ls in ((bt, K, V, lens), (pbt, Kp, Vp, priv)):
        kk, cu = wlmod.concat_rows(ks)
        vv, _ = wlmod.concat_rows(vs)
        if kk.shape[0]:
            m = max(max(ls), 1)
            binding.append(pool, 0, dev_bf16(kk), dev_bf16(vv), dev_i32(cu), dev_i32(table),
                           dev_i32(np.zeros(len(ls))), max_new=m, max_seq_len=m, dev_status=st)
    return dict(lens=list(lens), priv=list(priv), N=N, Hkv=Hkv, G=G, D=D, bt=bt, pbt=pbt,
                num_pages=num_pages, K=K, V=V, Kp=Kp, Vp=Vp, q=q, pool=pool, status=st, layer=0)


def run_decode_private(case, q_bits=None, priv=None, pbt=None, max_priv_len=None, scale=None):
    import torch

    q_bits = case["q"] if q_bits is None else q_bits
    priv = case["priv"] if priv is None else priv
    pbt = case["pbt"] if pbt is None else pbt
    B, N, Hq, D = q_bits.shape
    msl = max(max(case["lens"]), 1)
    mpl = max(max(priv), 0) if max_priv_len is None else max_priv_len
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    ws = nan_workspace(binding.decode_workspace_bytes(B, N, Hq, case["Hkv"], D, msl))
    out = torch.empty((B, N, Hq, D), dtype=torch.bfloat16, device="cuda")
    binding.decode_private(case["pool"], 0, dev_bf16(q_bits), out, dev_i32(case["bt"]), dev_i32(case["lens"]),
                           dev_i32(pbt), dev_i32(priv), msl, mpl, scale, ws, dev_status=case["status"])
    sync()
    return out


# Full-size parity: besides the absolute 2e-2, every sampled session's outputs
# must satisfy max|gpu - oracle| <= FULLSIZE_REL * max|oracle| (per session).
# tests/test_fullsize_bound.py shows on the CPU, with the oracle, that one
# dropped or duplicated 16-token page of an 8K-token context breaks this bound,
# while an emulation of the kernels' bf16 roundings (weights and outputs) stays
# well inside it.
FULLSIZE_REL = 1.0 / 64


def session_rel_err(got, want):
    """max|got - want| / max|want| over one session's outputs (float64 arrays)."""
    return float(np.max(np.abs(got - want))) / max(float(np.max(np.abs(want))), 1e-30)
