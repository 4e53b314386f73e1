"""The launch planner's split-KV chunk choice, on the CPU.

dab_plan.cpp holds no HIP code; it is built here with g++ (host sanitizers on) together with
tests/plan_host.cpp, which prints the plan of one configuration for a given number of compute units and
attention workgroups each holds at once (the library reads both from the HIP runtime).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_block_amd", "csrc")

PHASED, ATTN_OPROJ, AUTO = 1, 2, 0
BF16 = 1


@pytest.fixture(scope="module")
def plan_host(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path_factory.mktemp("plan") / "plan_host")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "plan_host.cpp"), os.path.join(CSRC, "dab_plan.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True)

    def run(B, H, nq, nkv, D, cap, schedule=AUTO, cus=0, per_cu=0, dtype=BF16, probe=0):
        out = subprocess.run([exe] + [str(v) for v in (B, H, nq, nkv, D, cap, dtype, schedule, cus, per_cu, probe)],
                             check=True, capture_output=True, text=True).stdout.split()
        st, sched, T, maxc, grid, split, worst, bad, at_probe = map(int, out)
        assert st == 0
        assert bad == 0 and worst <= maxc          # every position's chunks fit the grid and cover its tokens
        return dict(schedule=sched, T=T, max_chunks=maxc, grid=grid, split_merge=bool(split), worst=worst,
                    T_at=at_probe)
    run.exe = exe
    return run


def ffn_plan(plan_host, B, H, F, dtype=BF16):
    out = subprocess.run([plan_host.exe, "ffn", str(B), str(H), str(F), str(dtype)], check=True,
                         capture_output=True, text=True).stdout.split()
    vals = list(map(int, out))
    if len(vals) == 1:
        return dict(status=vals[0])
    keys = ["status", "mfma", "gu_tiles", "gu_panels", "gu_nb", "down_panels", "layout_ok", "hand_at",
            "ws_bytes", "check", "h_on_w_gate", "out_on_ws", "ws_on_fws", "w_gate_on_hidden"]
    return dict(zip(keys, vals))


def test_ffn_plan_and_layer_checks(plan_host):
    # the 7B FFN at batch 1 (VALU panels: 2752 gate/up panels of one feature per wave, 512 down panels)
    # and the 8B FFN at batch 16 (streamed gate/up panels of 7 mixed tiles, one 16-row down tile per CU);
    # the layout holds the overlapped layer's hand-off region after m and its bf16 copy, and the layer
    # call's check accepts disjoint arguments and rejects every written argument that overlaps another
    # half's (host sanitizers on)
    p7 = ffn_plan(plan_host, 1, 4096, 11008)
    assert (p7["status"], p7["mfma"], p7["gu_panels"], p7["gu_nb"], p7["down_panels"]) == (0, 0, 2752, 1, 512)
    p8 = ffn_plan(plan_host, 16, 4096, 14336)
    assert (p8["status"], p8["mfma"], p8["gu_tiles"], p8["gu_panels"], p8["down_panels"]) == (0, 1, 7, 256, 256)
    for p in (p7, p8, ffn_plan(plan_host, 3, 2048, 5632, dtype=0), ffn_plan(plan_host, 40, 4096, 14336)):
        assert p["status"] == 0 and p["layout_ok"] == 1
        assert p["check"] == 0
        assert p["h_on_w_gate"] == p["out_on_ws"] == p["ws_on_fws"] == 1      # DAB_ERR_INVALID_ARG
        assert p["w_gate_on_hidden"] == 0                                      # read-only inputs may coincide
    assert ffn_plan(plan_host, 1, 100, 11008)["status"] == 2          # DAB_ERR_UNSUPPORTED: H not a multiple of 64


def test_two_chunks_per_cu_beyond_one_round(plan_host):
    # 8B GQA layer, batch 16, 4K tokens: 1280 chunks of 448 tokens would need more than one round of
    # the 1024 resident workgroups (4 per CU x 256 CUs); two chunks per CU instead: 4 of 1024 tokens
    # per (sequence, kv head)
    p = plan_host(16, 4096, 32, 8, 128, 4097, cus=256, per_cu=4)
    assert p["schedule"] == PHASED and p["T"] == 1024 and p["max_chunks"] == 4 and p["grid"] == 512
    # three per CU: 768 resident, still more than one round; the same two per CU
    assert plan_host(16, 4096, 32, 8, 128, 4097, cus=256, per_cu=3)["grid"] == 512
    # without the device's figures: the device-free rule
    p0 = plan_host(16, 4096, 32, 8, 128, 4097)
    assert p0["T"] == 448 and p0["grid"] == 16 * 8 * 10


def test_one_head_per_kv_head_takes_whole_buffers(plan_host):
    # one query head per kv head: chunks are whole buffers of 128 tokens (D 128) or 256 (D 64)
    p = plan_host(1, 4096, 32, 32, 128, 1025, cus=256, per_cu=5)
    assert p["schedule"] == ATTN_OPROJ and p["T"] == 128 and p["grid"] == 256
    p = plan_host(1, 4096, 64, 64, 64, 1025, cus=256, per_cu=5)
    assert p["T"] == 256 and p["max_chunks"] == 4
    # grouped heads keep the plain rule: about 512 chunks, here 16 of 64 tokens per kv head (64 tokens
    # is the rule's lower limit at D 128)
    p = plan_host(1, 4096, 32, 8, 128, 1025, cus=256, per_cu=3)
    assert p["T"] == 64 and p["grid"] == 8 * 16


def test_residency_rule_leaves_other_shapes(plan_host):
    # 7B layer, batch 1: 512 chunks of 256 tokens fit one round; attention + projection in one launch
    p = plan_host(1, 4096, 32, 32, 128, 4097, cus=256, per_cu=5)
    assert p["schedule"] == ATTN_OPROJ and p["T"] == 256 and p["grid"] == 512
    # long context, batch 1: at most 64 chunks per kv head, 512 chunks fit one round
    p = plan_host(1, 4096, 32, 8, 128, 16385, cus=256, per_cu=3)
    assert p["T"] == 256 and p["max_chunks"] == 64 and p["split_merge"]
    # ragged batch 32 up to 8192 tokens: one round would need chunks over 1024 tokens; with a (sequence,
    # kv head) pair for every CU, 384-token chunks and no split of short sequences
    p = plan_host(32, 4096, 32, 8, 128, 8193, cus=256, per_cu=3)
    assert p["T"] == 384 and p["max_chunks"] == 22 and p["split_merge"]
    assert plan_host(32, 4096, 32, 8, 128, 8193, cus=256, per_cu=3, probe=300)["T_at"] == 304   # one chunk
    assert plan_host(16, 4096, 32, 8, 128, 8193, cus=256, per_cu=3, probe=300)["T_at"] == 80    # 128 pairs: four


def test_chunks_cover_every_cached_token(plan_host):
    for B, nkv, cap, per_cu in ((16, 8, 4097, 3), (3, 2, 1001, 3), (64, 8, 2049, 2), (8, 8, 30001, 4)):
        p = plan_host(B, 1024, 2 * nkv, nkv, 128, cap, cus=256, per_cu=per_cu)
        assert p["T"] % 16 == 0 and p["T"] * p["max_chunks"] >= cap - 1 > p["T"] * (p["max_chunks"] - 1)
        assert p["grid"] == B * nkv * p["max_chunks"]


def test_chunk_length_follows_the_position(plan_host):
    """A preallocated cache far larger than the context: the grid is sized for the capacity, and each
    sequence's chunks are sized for its own position, so a 4K context in a 32K cache gets the chunks a
    4K cache would give it."""
    big = plan_host(1, 4096, 32, 32, 128, 32768, cus=256, per_cu=5, probe=4096)
    small = plan_host(1, 4096, 32, 32, 128, 4097, cus=256, per_cu=5, probe=4096)
    assert big["T_at"] == small["T"] == 256
    assert big["max_chunks"] >= small["max_chunks"]
    # grouped heads and a batch: the same, the two-per-CU rule included (judged at the position: 4
    # chunks of 1024 tokens per kv head at 4K tokens in a 16K or 32K cache, as in a 4K cache)
    for cap in (16384, 32768):
        big = plan_host(16, 4096, 32, 8, 128, cap, cus=256, per_cu=4, probe=4096)
        small = plan_host(16, 4096, 32, 8, 128, 4097, cus=256, per_cu=4, probe=4096)
        assert big["T_at"] == small["T"] == 1024
    # other shapes and capacities: the walk over every position checks each plan
    for cap in (100, 2049, 65536):
        plan_host(3, 1024, 8, 2, 64, cap, cus=256, per_cu=3)
        plan_host(1, 1024, 8, 8, 128, cap, cus=0, per_cu=0)
