"""bench.py's host-side accounting, on the CPU: the per-kernel algorithmic bytes add up to the step's, the
rocprofv3 kernel names map to their phases, the committed counter summaries are read back, and a run
asked for more than one GPU stops before touching one."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from attention_block_amd.inputs import (CONFIGS, FFN_CONFIGS, MLA_CONFIGS, ffn_algorithmic_bytes,  # noqa: E402
                                        layer_ffn, mla_algorithmic_bytes, positions)


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_attention_phase_bytes_add_up(name):
    cfg = CONFIGS[name]
    pos = positions(cfg, 0)
    pb = bench.phase_bytes(cfg, pos)
    total = bench.algorithmic_bytes(cfg, pos)
    assert pb["qkv_rmsnorm_rope_append"] + pb["attention_split_kv"] + pb["oproj_residual"] == total
    assert pb["attention_oproj_residual"] == pb["attention_split_kv"] + pb["oproj_residual"]
    assert pb["qkv_attention_split_kv"] == pb["qkv_rmsnorm_rope_append"] + pb["attention_split_kv"]
    assert pb["decode_block_fused"] == total and pb["attention_merge"] == 0
    # the cache read is 2 (K and V) x kv heads x D x stored bytes x every cached token
    s = 2 if cfg.dtype == "bf16" else 4
    assert pb["attention_split_kv"] == 2 * cfg.n_kv_heads * cfg.head_dim * s * int(pos.sum())


@pytest.mark.parametrize("name", sorted(FFN_CONFIGS) + ["layer_ffn of " + n for n in sorted(CONFIGS)])
def test_ffn_phase_bytes_add_up(name):
    cfg = layer_ffn(CONFIGS[name.split()[-1]]) if name.startswith("layer_ffn") else FFN_CONFIGS[name]
    pb = bench.ffn_phase_bytes(cfg)
    assert sum(pb.values()) == ffn_algorithmic_bytes(cfg)
    s = 2 if cfg.dtype == "bf16" else 4
    # the weights dominate: W_gate and W_up with the first kernel, W_down with the second
    assert pb["ffn_rmsnorm_gate_up_silu"] >= 2 * s * cfg.hidden * cfg.intermediate
    assert pb["ffn_down_residual"] >= s * cfg.hidden * cfg.intermediate


@pytest.mark.parametrize("name", sorted(MLA_CONFIGS))
def test_mla_phase_bytes(name):
    import numpy as np
    cfg = MLA_CONFIGS[name]
    pos = np.full(cfg.batch, cfg.pos)                 # every sequence at the workload's position
    pb = bench.mla_phase_bytes(cfg, pos)
    assert pb["mla_merge"] == 0 and pb["mla_chunk"] == mla_algorithmic_bytes(cfg, pos)
    # at least the latent and rotary rows of every cached token, once
    s = 2 if cfg.dtype == "bf16" else 4
    assert pb["mla_chunk"] >= s * (cfg.kv_lora_rank + cfg.rope_dim) * int(pos.sum())


@pytest.mark.parametrize("kernel,phase", [
    ("void dab::dev::qkv_kernel<unsigned short, 1, true>(dab::StepArgs)", "qkv_rmsnorm_rope_append"),
    ("void dab::dev::attn_oproj_kernel<unsigned short, 128, 1, 1>(dab::StepArgs)", "attention_oproj_residual"),
    ("void dab::dev::mfma_str_kernel<true, 1, 1, 4>(dab::StepArgs)", "qkv_rmsnorm_rope_append"),
    ("void dab::dev::mfma_str_kernel<false, 1, 1, 4>(dab::StepArgs)", "oproj_residual"),
    ("void dab::dev::mfma_str_qkv24_kernel<1, 4>(dab::StepArgs)", "qkv_rmsnorm_rope_append"),
    ("void dab::dev::(anonymous namespace)::ffn_str_kernel<7, 1, 4>(dab::FfnArgs)", "ffn_rmsnorm_gate_up_silu"),
    ("void dab::dev::(anonymous namespace)::ffn_str_down_kernel<1, 14>(dab::FfnArgs)", "ffn_down_residual"),
    ("void dab::dev::(anonymous namespace)::ffn_down_kernel<unsigned short, 1, false, 3>(dab::FfnArgs)",
     "ffn_down_residual"),
    ("void dab::dev::(anonymous namespace)::ffn_mfma_kernel<true, 2, 1>(dab::FfnArgs)", "ffn_rmsnorm_gate_up_silu"),
    ("void dab::dev::(anonymous namespace)::ffn_mfma_kernel<false, 1, 1>(dab::FfnArgs)", "ffn_down_residual"),
    ("elementwise_copy", None),
])
def test_kernel_names_map_to_phases(kernel, phase):
    assert bench.phase_of(kernel) == phase


def test_committed_counter_summaries_are_read_back():
    # every committed FETCH_SIZE / WRITE_SIZE summary names its kernel's phase and workload; its traffic is
    # reported only for the kernel sources it was taken on
    names = [f for f in os.listdir(bench.PROFILES) if f.startswith("pmc_traffic_")]
    assert names
    current = bench.source_digest()
    for f in names:
        text = open(os.path.join(bench.PROFILES, f)).read()
        assert "source_digest:" in text and "hbm_bytes_per_launch:" in text, f
        phase, workload = None, None
        for ph in sorted(set(p for _, p in bench.KERNEL_PHASES) | {"oproj_residual", "ffn_down_residual"},
                         key=len, reverse=True):
            if f.startswith(f"pmc_traffic_{ph}_"):
                phase, workload = ph, f[len(f"pmc_traffic_{ph}_"):-len(".md")]
                break
        assert phase is not None, f
        got = bench.measured_traffic(phase, workload)
        if f"`{current}`" in text:
            assert isinstance(got, int) and got > 0, f
        else:
            assert got is None, f
    assert bench.measured_traffic("qkv_rmsnorm_rope_append", "no_such_workload") is None


def test_host_cores_are_the_affinity_set():
    assert bench.host_cpu()["cores"] == len(os.sched_getaffinity(0))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single" in r.stderr
