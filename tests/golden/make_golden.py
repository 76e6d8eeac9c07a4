"""Writes the hand-worked fixtures in this folder.

Every expected value here is a closed form derived by hand (the derivation is
stored next to it); the pages print no numeric example.  Nothing here calls the
oracle or the GPU library.  Run: python tests/golden/make_golden.py
"""
import json
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def dump(name, obj):
    with open(os.path.join(HERE, name), "w") as f:
        json.dump(obj, f, indent=1)
        f.write("\n")


def main():
    dump("route_example.json", {
        "citation": "Constructed worked example (the pages print none). Router of the fused-MoE interface named in "
                    "'Marlin moe integration' (nm-vllm PR 266), review comment on the fused_moe interface.",
        "derivation": "exp(logits - max) = [1/4, 2/4, 3/4, 4/4]; top-2 ids by descending logit = [3, 2]. "
                      "renormalize: w = [4/7, 3/7]. Full softmax: denominator 10/4, w = [4/10, 3/10].",
        "logits": [0.0, math.log(2.0), math.log(3.0), math.log(4.0)],
        "topk": 2,
        "ids": [3, 2],
        "weights_renorm": [4 / 7, 3 / 7],
        "weights_full_softmax": [0.4, 0.3],
    })
    dump("align_example.json", {
        "citation": "Constructed worked example of the token sort and pad per expert (moe_align_block_size) named in "
                    "'Marlin moe integration' (nm-vllm PR 266), review thread on moe_align_block_size_kernel and the "
                    "hard-coded block size.",
        "derivation": "flattened ids [2,0,0,1,1,2] (i = m*topk+j); counts e0:{1,2} e1:{3,4} e2:{0,5} e3:{}; block 4 "
                      "pads each to 4; offsets 0,4,8; sentinel = M*topk = 6; capacity = 6 + min(4,6)*3 = 18 -> 20.",
        "topk_ids": [[2, 0], [0, 1], [1, 2]], "E": 4, "block_size": 4,
        "capacity": 20,
        "sorted_token_ids": [1, 2, 6, 6, 3, 4, 6, 6, 0, 5, 6, 6, 6, 6, 6, 6, 6, 6, 6, 6],
        "expert_ids": [0, 1, 2, -1, -1],
        "num_tokens_post_padded": 12,
    })
    h0 = 1.0 / (1.0 + math.exp(-1.0)) * 2.0   # gate 1, up 2
    h1 = 1.5 / (1.0 + math.exp(-1.5)) * 3.0   # gate 1.5, up 3
    y0 = [h0, h0]
    y1 = [h1, -0.5 * h1]
    dump("layer_example.json", {
        "citation": "Constructed worked example of the fused MoE layer with per-column symmetric int8 weights as "
                    "described in the opening of '[Kernel] W8A16 Int8 inside FusedMoE' (vLLM PR 7415): weights times "
                    "their per-output-column scale, SiLU(gate)*up between the projections, top-k weighted sum.",
        "derivation": [
            "x = [1, 2]; logits = [0, ln 3] -> slots: expert 1 (w = 3/4), expert 0 (w = 1/4)",
            "expert 0: gate row q=[1,0] s=1 -> gate = 1; up row q=[0,1] s=1 -> up = 2; h0 = silu(1)*2 = 2/(1+e^-1)",
            "expert 0: W2 = [[1],[1]] (q=[[1],[1]], s=1) -> y0 = [h0, h0]",
            "expert 1: gate row q=[1,1] s=0.5 -> gate = 1.5; up row q=[1,1] s=1 -> up = 3; "
            "h1 = silu(1.5)*3 = 4.5/(1+e^-1.5)",
            "expert 1: W2 q=[[4],[-2]] s=0.25 -> [[1],[-0.5]] -> y1 = [h1, -0.5 h1]",
            "out = 3/4 y1 + 1/4 y0"],
        "x": [[1.0, 2.0]], "logits": [[0.0, math.log(3.0)]], "topk": 2,
        "w1q": [[[1, 0], [0, 1]], [[1, 1], [1, 1]]],
        "s1": [[[1.0, 1.0]], [[0.5, 1.0]]],
        "w2q": [[[1], [1]], [[4], [-2]]],
        "s2": [[[1.0, 1.0]], [[0.25, 0.25]]],
        "ids": [[1, 0]], "weights": [[0.75, 0.25]],
        "gu": [[1.5, 3.0], [1.0, 2.0]],
        "h": [[h1], [h0]], "y": [y1, y0], "out": [[0.75 * y1[c] + 0.25 * y0[c] for c in range(2)]],
    })
    dump("actorder_example.json", {
        "citation": "Constructed example of GPTQ act-order ('Marlin moe integration', nm-vllm PR 266, end-to-end "
                    "test description with the gptq-4bit-128g-actorder checkpoint): input channel k belongs to scale "
                    "group g_idx[k], not k // group_size.",
        "derivation": "K=4, group size 2, g_idx = [1,0,0,1]; scales group0 = 1, group1 = 2 for both rows; gate row "
                      "q = [1,1,1,1] -> W = [2,1,1,2]; up row q = [3,0,0,-1] -> W = [6,0,0,-2]; x = [1,0,0,0] -> "
                      "gate = 2, up = 6 (ignoring g_idx would give 1 and 3).",
        "x": [[1.0, 0.0, 0.0, 0.0]], "g_idx": [[1, 0, 0, 1]],
        "w1q": [[[1, 1, 1, 1], [3, 0, 0, -1]]], "s1": [[[1.0, 1.0], [2.0, 2.0]]],
        "gu": [[2.0, 6.0]],
    })
    dump("sparse_example.json", {
        "citation": "Constructed example of a 2:4-structured-sparse 4-bit row with group scales ('Add GPTQ Marlin "
                    "2:4 sparse structured support', vLLM PR 4790, opening description: 2:4 sparsity, 4-bit, group "
                    "size 128 -- here group size 4 to keep it tiny).",
        "derivation": "K=8, group size 4; group 0 keeps positions (1,3) codes (2,-3) scale 0.5; group 1 keeps (0,2) "
                      "codes (1,5) scale 0.25; x = [1..8]; y = 2*2*0.5 + 4*(-3)*0.5 + 5*1*0.25 + 7*5*0.25 = 6",
        "x": [[1, 2, 3, 4, 5, 6, 7, 8]], "vals": [[2, -3, 1, 5]], "idx": [[1, 3, 0, 2]], "s": [[0.5], [0.25]],
        "group_size": 4,
        "y": [[6.0]],
    })


if __name__ == "__main__":
    main()
