"""Host logic of bench.py: the source digest that ties a counter summary to the
kernel code it was taken on."""

import bench

SRC = """// a kernel
__global__ void k(float* x) {   /* one lane */
  x[threadIdx.x] = x[threadIdx.x] + 1.0f;  // add one
}
"""


def test_digest_ignores_comments_and_blank_space():
    d = bench.code_digest([SRC])
    assert bench.code_digest([SRC.replace("// add one", "// add 1 to each element")]) == d
    assert bench.code_digest([SRC.replace("/* one lane */", "/* one lane,\n   one element */")]) == d
    assert bench.code_digest([SRC.replace("  x[", "\n\n      x[")]) == d
    assert bench.code_digest(["// header\n" + SRC]) == d


def test_digest_changes_with_the_code():
    d = bench.code_digest([SRC])
    assert bench.code_digest([SRC.replace("1.0f", "2.0f")]) != d
    assert bench.code_digest([SRC.replace("+ 1.0f", "- 1.0f")]) != d
    assert bench.code_digest([SRC, "int y;"]) != d
