"""dflash2_verify_greedy_noalloc (greedy verification with a fixed device
scratch array instead of a workspace) against dflash2_verify_greedy with a
workspace, through the C ABI: bit-identical accept lengths and emitted
tokens on two calls in a row, the second smaller than the first, and the
oracle's greedy verification on both."""
import ctypes as C

import numpy as np
import pytest
import torch

import draft_selection_bf16_amd as df2
import oracle
import synth

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _case(B, T, V, seed, dtype=torch.bfloat16):
    dev = torch.device("cuda:0")
    w = synth.scaled(synth.WORKLOADS["b32_blk16_v151936_conv"], B=B, block=T + 1, V=V, seed=seed)
    z, tok, _ = synth.drafter_logits(w, device=dev)
    Z = synth.target_logits(w, z, tok, device=dev).to(dtype).contiguous()
    g = torch.Generator(device=dev).manual_seed(seed)
    flip = torch.rand(tok.shape, generator=g, device=dev) < 0.2
    path = torch.where(flip, (tok + 1) % V, tok).to(torch.int32).contiguous()
    return Z, path


def _run(Z, path, noalloc):
    L = df2.lib()
    B, T1, V = Z.shape
    dev = Z.device
    acc = torch.full((B,), -9, dtype=torch.int32, device=dev)
    out = torch.full((B, T1), -9, dtype=torch.int32, device=dev)
    s = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t: C.c_void_p(t.data_ptr())
    dt = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}[Z.dtype]
    if noalloc:
        st = L.dflash2_verify_greedy_noalloc(p(Z), dt, V, p(path), B, T1 - 1, p(acc), p(out), s)
    else:
        need = L.dflash2_verify_workspace_bytes(B, T1 - 1, V)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        st = L.dflash2_verify_greedy(p(Z), dt, V, p(path), B, T1 - 1, p(acc), p(out), p(ws), need, s)
    assert st == 0, L.dflash2_last_error()
    torch.cuda.synchronize()
    return acc.cpu().numpy(), out.cpu().numpy()


def test_noalloc_greedy_verify_matches_workspace_entry_point():
    L = df2.lib()
    L.dflash2_verify_greedy_noalloc.argtypes = [C.c_void_p, C.c_int, C.c_int64, C.c_void_p, C.c_int, C.c_int,
                                                 C.c_void_p, C.c_void_p, C.c_void_p]
    L.dflash2_verify_greedy_noalloc.restype = C.c_int
    L.dflash2_verify_greedy_noalloc_max_bytes.restype = C.c_size_t
    assert L.dflash2_verify_greedy_noalloc_max_bytes() == 1 << 20
    # a larger call, then a smaller one that reuses the same scratch
    for B, T, V, seed in ((32, 15, 151936, 21), (3, 7, 50021, 22)):
        print(f"[case] noalloc greedy verify B={B} T={T} V={V}", flush=True)
        Z, path = _case(B, T, V, seed)
        a_ws, o_ws = _run(Z, path, noalloc=False)
        a_na, o_na = _run(Z, path, noalloc=True)
        assert np.array_equal(a_na, a_ws) and np.array_equal(o_na, o_ws)
        ov = oracle.verify_greedy(Z.cpu(), path.cpu())
        assert np.array_equal(a_na, ov["accept_len"]) and np.array_equal(o_na, ov["out_tok"])
        print(f"[parity] noalloc greedy verify B={B}: mean_accept={float(a_na.mean()):.3f}", flush=True)
