"""Hot calls allocate nothing and never synchronise: a static check on the
built library.

The host code of libq4k.so is disassembled (objdump) into a call graph of
direct calls (PLT stubs resolved to the symbol they stand for).  From every
hot entry point no path may reach a HIP routine that allocates or frees
device memory, clears it with a blocking call, or waits for the device.
Plan creation is the one place that does all of that, which the last test
checks so that the analysis is known to see such calls at all.
"""
from __future__ import annotations

import collections
import re
import subprocess

import pytest

import bit_block_quantized_gguf_amd as q4k

HOT = ("q4k_dequant", "q4k_gemv", "q4k_gemv_batch", "q4k_gemm", "q4k_gemv_q8_0",
       "q4k_gemv_q6_k", "q4k_mlp", "q4k_workspace_size", "q4k_decode_stack",
       "q4k_decode_stack_buffer", "q4k_decode_stack_nodes", "q4k_gemv_noalloc",
       "q4k_gdn_step", "q4k_attn_step", "q4k_decode_stack_reset",
       "q4k_decode_stack_position")
FORBIDDEN = re.compile(r"^(hipMalloc\w*|hipExtMalloc\w*|hipHostMalloc|hipMallocManaged|hipFree\w*|"
                       r"hipHostFree|hipMemset|hipMemsetD\w*|hipDeviceSynchronize|"
                       r"hipStreamSynchronize|hipEventSynchronize|hipMemcpy|hipGraphInstantiate\w*|"
                       r"hipStreamBeginCapture|hipGraphUpload)$")


@pytest.fixture(scope="module")
def graph():
    out = subprocess.run(["objdump", "-d", "--no-show-raw-insn", q4k.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    calls = collections.defaultdict(set)
    cur = None
    for line in out.splitlines():
        m = re.match(r"^[0-9a-f]+ <([^>]+)>:$", line)
        if m:
            cur = m.group(1)
            continue
        m = re.search(r"\s(?:call|jmp)\s+[0-9a-f]+ <([^>+]+)(?:\+0x[0-9a-f]+)?>", line)
        if m and cur:
            callee = m.group(1)
            if callee.endswith("@plt"):
                callee = callee[:-4]
            if callee != cur:
                calls[cur].add(callee)
    return calls


def _reach(graph, root):
    seen, todo, parent = {root}, [root], {}
    while todo:
        f = todo.pop()
        for g in graph.get(f, ()):
            if g not in seen:
                seen.add(g)
                parent[g] = f
                todo.append(g)
    return seen, parent


@pytest.mark.parametrize("entry", HOT)
def test_hot_entry_reaches_no_allocation_or_wait(graph, entry):
    assert entry in graph, entry
    seen, parent = _reach(graph, entry)
    bad = sorted(f for f in seen if FORBIDDEN.match(f))
    if bad:
        chain, f = [bad[0]], bad[0]
        while f in parent:
            f = parent[f]
            chain.append(f)
        pytest.fail("%s reaches %s via %s" % (entry, bad, " <- ".join(chain)))


def test_analysis_sees_plan_creation_allocate(graph):
    seen, _ = _reach(graph, "q4k_decode_stack_create")
    assert "hipMalloc" in seen and "hipGraphInstantiate" in seen
