"""Helpers of the GPU parity tests: run the HIP path through the C ABI and read
results back for comparison with the oracle. Nothing here computes the method."""
import sys

import numpy as np

PLAN_INT_KEYS = ("status", "T", "hoff", "L", "keep", "O", "D", "Opre", "Dpre", "dst", "src",
                 "n_dup", "dup_expert", "dup_start", "dup_count", "seg_ptr", "seg_expert",
                 "n_list", "list_expert", "list_rank", "list_b", "dup_ptr")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dims_for(td, R, E, K, S, B, H, dtype):
    return td.Dims(R, E, K, S, B, dtype, H)


def run_plan(td, dims, ids_np, dev, plan_buf=None, bounded=False, form=None):
    """Plan through the C ABI: moonep_plan / moonep_plan_bounded, or with form
    "two" / "four" the launch form forced through moonep_plan_ex."""
    import torch
    if plan_buf is None:
        plan_buf = td.new_plan_buffer(dims, dev)
    ids_d = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).to(dev)
    if form is None:
        (td.moonep_plan_bounded if bounded else td.moonep_plan)(dims, ids_d, plan_buf)
    else:
        flags = {"two": td.PLAN_TWO_LAUNCH, "four": td.PLAN_FOUR_LAUNCH}[form]
        td.moonep_plan_ex(dims, ids_d, plan_buf, flags | (td.PLAN_BOUNDED if bounded else 0))
    torch.cuda.synchronize()
    return plan_buf, ids_d


def other_form(td, dims):
    """The launch form moonep_plan does not take for these dims."""
    return "four" if td.moonep_plan_layout(dims).plan_launches == 2 else "two"


def read_plan(td, dims, plan_buf):
    v = td.plan_views(dims, plan_buf)
    out = {k: t.cpu().numpy() for k, t in v.items()}
    out["dcap"] = out["dup_expert"].shape[1]
    return out


def assert_plan_equal(gpu, orc):
    """Bit-exact comparison of every public plan array."""
    for k in PLAN_INT_KEYS:
        g = np.asarray(gpu[k]).reshape(-1).astype(np.int64)
        o = np.asarray(orc[k]).reshape(-1).astype(np.int64)
        if not np.array_equal(g, o):
            bad = np.nonzero(g != o)[0] if g.shape == o.shape else None
            raise AssertionError(
                f"plan array {k} differs: shapes {g.shape} vs {o.shape}; "
                f"first mismatches at {None if bad is None else bad[:8].tolist()}: "
                f"gpu {None if bad is None else g[bad[:8]].tolist()} "
                f"oracle {None if bad is None else o[bad[:8]].tolist()}")
    assert int(np.asarray(gpu["maxT"]).reshape(-1)[0]) == int(np.asarray(orc["maxT"]).reshape(-1)[0])
    gm = np.asarray(gpu["maxvio"]).reshape(-1)[:1].view(np.uint64)
    om = np.asarray(orc["maxvio"]).reshape(-1)[:1].view(np.uint64)
    assert np.array_equal(gm, om), "maxvio bits differ"


def bf16_bits(t):
    """uint16 numpy view of a bf16 torch tensor (CPU copy)."""
    import torch
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def f32_bits(t):
    return t.detach().contiguous().cpu().numpy().view(np.uint32)


class HostStage:
    """A pinned host buffer through which device tensors are copied to the host in
    batches; fetch() returns a numpy view that is valid until the next fetch."""

    def __init__(self, nbytes: int):
        import torch
        self.buf = torch.empty(max(16, int(nbytes)), dtype=torch.uint8, pin_memory=True)

    def fetch(self, t):
        import torch
        t = t.contiguous()
        n = t.numel() * t.element_size()
        assert n <= self.buf.numel(), f"stage of {self.buf.numel()} bytes, needs {n}"
        h = self.buf[:n].view(t.dtype).view(t.shape)
        h.copy_(t)
        if t.dtype == torch.bfloat16:
            return h.view(torch.int16).numpy().view(np.uint16)
        return h.numpy()


def token_batches(n_tok: int, K: int, row_bytes: int, budget: int = 1 << 30):
    """Token ranges [t0, t0 + n) whose K gathered rows take at most `budget` bytes."""
    tb = max(1, min(n_tok, budget // (K * row_bytes)))
    for t0 in range(0, n_tok, tb):
        yield t0, min(tb, n_tok - t0)


def local_dst(dst_tokens: np.ndarray) -> np.ndarray:
    """Entry a of a batch reads gathered row a; dropped entries stay -1."""
    d = np.arange(dst_tokens.size, dtype=np.int32)
    d[dst_tokens.reshape(-1) < 0] = -1
    return d
