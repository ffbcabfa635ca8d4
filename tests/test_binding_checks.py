"""Host-side argument checks of the Python binding (no GPU needed).

The C ABI receives bare device pointers and cannot see buffer sizes, so the binding checks every
tensor against the sizes and ``fmt`` of the call before anything reaches the library: a buffer
that is too small, or an output of the wrong type, must raise ValueError. These tests call the
checkers directly with CPU tensors of the right and the wrong sizes."""

import pytest
import torch

import mx_grouped_gemm_amd as bsg

M, N, K, E, T = 256, 384, 512, 3, 2


def blockwise(**over):
    a = dict(A=torch.zeros(M, K, dtype=torch.uint8), a_scales=torch.ones(M, K // 128),
             B=torch.zeros(E, N, K, dtype=torch.uint8), b_scales=torch.ones(E, N // 128, K // 128),
             expert_ids=torch.zeros(T, dtype=torch.int32),
             tile_offsets=torch.zeros(T + 1, dtype=torch.int32),
             C=torch.zeros(M, N, dtype=torch.bfloat16), M=M, N=N, K=K,
             fmt=bsg.make_fmt("e4m3", "e4m3", "blockwise", "bf16"), num_tiles=T, num_experts=E)
    a.update(over)
    return a


def test_valid_blockwise_call_passes():
    bsg.check_grouped_args(**blockwise())


@pytest.mark.parametrize("over,msg", [
    (dict(C=torch.zeros(M, N, dtype=torch.float32)), "C must be"),                 # f32 buffer, bf16 fmt
    (dict(fmt=bsg.make_fmt("e4m3", "e4m3", "blockwise", "f32")), "C must be"),      # bf16 buffer, f32 fmt
    (dict(C=torch.zeros(M - 1, N, dtype=torch.bfloat16)), "C holds"),
    (dict(M=M + 128), "A holds"),                                                   # M past A's rows
    (dict(A=torch.zeros(M, K // 2, dtype=torch.uint8)), "A holds"),
    (dict(a_scales=torch.ones(M, K // 128 - 1)), "a_scales holds"),
    (dict(a_scales=torch.ones(M, K // 128, dtype=torch.float16)), "a_scales must be float32"),
    (dict(B=torch.zeros(E - 1, N, K, dtype=torch.uint8)), "B holds"),
    (dict(b_scales=torch.ones(E, N // 128, K // 128 - 1)), "b_scales holds"),
    (dict(expert_ids=torch.zeros(T - 1, dtype=torch.int32)), "expert_ids holds"),
    (dict(tile_offsets=torch.zeros(T, dtype=torch.int32)), "tile_offsets holds"),
    (dict(expert_ids=torch.zeros(T, dtype=torch.int64)), "expert_ids must be int32"),
    (dict(tile_offsets=None), "both given or both None"),
    (dict(A=torch.zeros(M, K, dtype=torch.float32)), "one byte per element"),
])
def test_blockwise_mismatch_raises(over, msg):
    with pytest.raises(ValueError, match=msg):
        bsg.check_grouped_args(**blockwise(**over))


def test_dense_call_needs_one_expert_of_b():
    a = blockwise(expert_ids=None, tile_offsets=None, B=torch.zeros(1, N, K, dtype=torch.uint8),
                  b_scales=torch.ones(1, N // 128, K // 128))
    bsg.check_grouped_args(**a)
    a["B"] = torch.zeros(N - 128, K, dtype=torch.uint8)
    with pytest.raises(ValueError, match="B holds"):
        bsg.check_grouped_args(**a)


@pytest.mark.parametrize("fa,fb,kind,per", [("e4m3", "e2m1", "mx", 32), ("e2m1", "e2m1", "mx", 32),
                                            ("e2m1", "e2m1", "nv", 16)])
def test_mx_and_nv_layouts(fa, fb, kind, per):
    ra = K if fa == "e4m3" else K // 2
    rb = K if fb == "e4m3" else K // 2
    a = dict(A=torch.zeros(M, ra, dtype=torch.uint8), a_scales=torch.zeros(M, K // per, dtype=torch.uint8),
             B=torch.zeros(1, N, rb, dtype=torch.uint8), b_scales=torch.zeros(1, N, K // per, dtype=torch.uint8),
             expert_ids=None, tile_offsets=None, C=torch.zeros(M, N, dtype=torch.float16), M=M, N=N, K=K,
             fmt=bsg.make_fmt(fa, fb, kind, "f16"), num_tiles=0, num_experts=1)
    bsg.check_grouped_args(**a)
    for name, bad in (("a_scales", torch.zeros(M, K // per - 1, dtype=torch.uint8)),
                      ("b_scales", torch.zeros(1, N, K // per - 1, dtype=torch.uint8)),
                      ("A", torch.zeros(M, ra - 16, dtype=torch.uint8)),
                      ("B", torch.zeros(1, N, rb - 16, dtype=torch.uint8))):
        with pytest.raises(ValueError, match=f"{name} holds"):
            bsg.check_grouped_args(**{**a, name: bad})


def test_sizes_the_library_rejects_are_left_to_it():
    # N not a multiple of 128, a negative M and an unknown scale kind: the library returns a
    # status for these, so the checker does not second-guess them
    bsg.check_grouped_args(**blockwise(N=100))
    bsg.check_grouped_args(**blockwise(M=-1))
    bsg.check_grouped_args(**blockwise(fmt=bsg.make_fmt("e4m3", "e4m3", "blockwise", "bf16") | (7 << 8)))


def permute_args(**over):
    tokens, top_k, Mp = 64, 4, 512
    a = dict(x=torch.zeros(tokens, K, dtype=torch.bfloat16), topk_ids=torch.zeros(tokens, top_k, dtype=torch.int32),
             expert_offsets=torch.zeros(E + 1, dtype=torch.int32), M=Mp, num_experts=E,
             dest=torch.zeros(tokens, top_k, dtype=torch.int32), qa=torch.zeros(Mp, K, dtype=torch.uint8),
             a_scales=torch.zeros(Mp, K // 128))
    a.update(over)
    return a


def test_permute_checks():
    bsg.check_permute_args(**permute_args())
    for over, msg in ((dict(qa=torch.zeros(511, K, dtype=torch.uint8)), "qa must be"),
                      (dict(a_scales=torch.zeros(512, K // 128 - 1)), "a_scales must be"),
                      (dict(a_scales=torch.zeros(512, K // 128, dtype=torch.float64)), "a_scales must be float32"),
                      (dict(dest=torch.zeros(63, 4, dtype=torch.int32)), "dest holds"),
                      (dict(expert_offsets=torch.zeros(E, dtype=torch.int32)), "expert_offsets holds"),
                      (dict(topk_ids=torch.zeros(63, 4, dtype=torch.int32)), "topk_ids must be"),
                      (dict(x=torch.zeros(64 * K, dtype=torch.bfloat16)), "x must be")):
        with pytest.raises(ValueError, match=msg):
            bsg.check_permute_args(**permute_args(**over))
