"""Host logic of bench.py (no GPU): the one-GPU contract and the source
fingerprint that decides whether the committed HBM counters still describe
the kernels."""
import os
import subprocess
import sys

import bench  # noqa: F401  (importable without a GPU)
from block_causal_attention_qi_amd.profile_summary import kernel_code_text, kind_of, label_launches

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    assert r.returncode == 2
    assert r.stdout == ""
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr


def test_kernel_fingerprint_ignores_comments_and_layout_only():
    src = "int f(int a) {\n  // scale\n  return a * 2; /* twice */\n}\n"
    same = "int f(int a) { /* other words */ return a * 2;   // changed comment\n}"
    other = "int f(int a) {\n  // scale\n  return a * 3; /* twice */\n}\n"
    assert kernel_code_text(src) == kernel_code_text(same)
    assert kernel_code_text(src) != kernel_code_text(other)
    assert "scale" not in kernel_code_text(src)  # the comments are gone


def test_committed_counter_summary_names_its_fingerprint_and_kernels():
    import json
    rec = json.load(open(os.path.join(ROOT, "profiles", "dit32_1024px_hbm_traffic.json")))
    assert len(rec["kernel_source_sha256"]) == 64
    for kind in ("gemm_gate_up", "gemm_qkv", "gemm_down", "gemm_o", "attention"):
        ent = rec["kernels"][kind]["image-only"]
        assert int(ent["hbm_bytes"]) > 0


def test_profile_summary_classifies_launches_by_name_and_step():
    assert kind_of("void gemm_bf16_lds_kernel<1, 256, 256, 8>(GemmArgs)", "attention") == "gemm_o"
    assert kind_of("void gemm_bf16_mid_kernel<1>(GemmArgs)", "gemm_o") == "gemm_o"  # the O-proj's row tail
    assert kind_of("void gemm_bf16_lds_kernel<1, 256, 256, 8>(GemmArgs)", "gemm_gate_up") == "gemm_down"
    assert kind_of("void gemm_bf16_large_kernel<3, 2, 4, 128>(GemmArgs)", None) == "gemm_qkv"
    assert kind_of("void gemm_bf16_kernel<0, 128, 128>(GemmArgs)", None) == "gemm_txt"
    assert kind_of("void block_causal_attn_kernel<8>(AttnBatch)", None) == "attention"
    assert kind_of("void rmsnorm_mod_kernel<16>(float const*)", None) == "norm_mod"
    # a joint step (it runs the text projection; its first norm is the text norm), then an
    # image-only step; the joint pass splits the O-proj into a head and a row tail
    joint = ["mod_gemv_kernel<8>", "rmsnorm_mod_kernel<16>", "gemm_bf16_kernel<0, 128, 128>", "img_embed_kernel<4>",
             "rmsnorm_mod_kernel<16>", "gemm_bf16_lds_kernel<3, 256, 256, 8>", "block_causal_attn_kernel<8>",
             "gemm_bf16_lds_kernel<1, 256, 256, 8>", "gemm_bf16_mid_kernel<1>", "head_kernel<2>", "euler_kernel"]
    img = ["mod_gemv_kernel<8>", "img_embed_kernel<4>", "rmsnorm_mod_kernel<16>", "gemm_bf16_lds_kernel<3, 256, 256, 8>",
           "block_causal_attn_kernel<8>", "gemm_bf16_lds_kernel<1, 256, 256, 8>", "head_kernel<2>", "euler_kernel"]
    lab = label_launches(joint + img)
    assert lab[1] == ("norm_mod", "joint (text)") and lab[2] == ("gemm_txt", "joint (text)")
    assert lab[4] == ("norm_mod", "joint")
    assert lab[7] == ("gemm_o", "joint") and lab[8] == ("gemm_o", "joint")
    assert all(p == "image-only" for _, p in lab[len(joint):])
    assert [k for k, _ in lab[len(joint):]] == ["modulation", "img_embed", "norm_mod", "gemm_qkv", "attention",
                                                  "gemm_o", "head", "euler"]

