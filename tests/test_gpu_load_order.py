"""The binding works when the library is loaded before anything has imported torch.

torch ships its own HIP runtime; the library must bind to that one, whose device
memory and streams the binding hands over.  A fresh process loads the library as
its very first step, then runs the pages' 100-token request through
paged_attn_decode and checks it against the oracle.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, %r)
from paged_kv_cache_280_amd import _binding
_binding.load_library()  # first thing the process does
import numpy as np
import torch
import oracle
import paged_kv_cache_280_amd as pkv
import workloads as wl
case = wl.case_tiny(0)
q = wl.host_q(case)
kp, vp = wl.host_pools(case)
ref = oracle.paged_decode(q, kp, vp, case.block_tables, case.context_lens, case.block_size,
                          case.scale, case.num_kv_heads)
dev = torch.device("cuda:0")
to = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
out = pkv.paged_attn_decode(to(q), to(kp), to(vp), torch.from_numpy(case.block_tables).to(dev),
                            torch.from_numpy(case.context_lens).to(dev), case.block_size, case.scale,
                            max_context_len=case.max_context_len)
torch.cuda.synchronize()
err = np.abs(out.float().cpu().numpy() - ref)
print("max_abs %%.3g mean_abs %%.3g" %% (err.max(), err.mean()), flush=True)
assert err.max() <= 1e-2 and err.mean() <= 1e-3
print("ok", flush=True)
""" % ROOT


@pytest.mark.gpu
def test_library_loaded_before_torch():
    res = subprocess.run([sys.executable, "-c", CHILD], stdout=subprocess.PIPE,
                         stderr=subprocess.STDOUT, text=True, timeout=110)
    print(res.stdout[-2000:])
    assert res.returncode == 0 and res.stdout.strip().endswith("ok")
